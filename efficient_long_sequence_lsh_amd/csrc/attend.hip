// Stages 3 + 4: gather sorted rows and run chunked attention for every round.
//
// "Reformer: The Efficient Transformer" (research summary), Key points:
//   LSH attention bullet -- after sorting, each chunk of m positions attends to
//   itself and to the chunk before it;
//   Shared-QK bullet -- queries and keys are the same vectors, and a token does
//   not attend to itself unless it has no other valid target (the fallback is
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

namespace rlsh {

namespace {

constexpr int kQTile = 64;       // sorted slots per query tile (4 waves x 16)
constexpr int kKTile = 64;       // sorted slots per key tile
constexpr int kRunTiles = 4;     // query tiles per workgroup

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
struct AttnLds<D, true> {
  static constexpr int kKPitch = D + 8;      // bf16 elements per K row (16-byte pad)
  static constexpr int kVPitch = kKTile + 4; // bf16 elements per transposed V row
  uint16_t k[kKTile * kKPitch];
  uint16_t vt[D * kVPitch];
  int kpos[kKTile];
};

template <int D>
struct AttnLds<D, false> {
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
                                                           float* __restrict__ o_rounds, float* __restrict__ z_rounds) {
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

  const int qt_begin = blockIdx.x * kRunTiles;
  const int qt_end = min(s.n_qt, qt_begin + kRunTiles);

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
      const float alpha = exp2f(m_run - m_use);     // 0 when m_run = -inf
      float psum = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = exp2f(sc[t][j] - m_use);   // exp2(-inf) = 0 for masked keys
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

template <int D, bool BF16>
hipError_t launch_typed(const void* qk, const void* v, const int32_t* perm, int n_seg, AttnShape s, float* o, float* z,
                        hipStream_t stream) {
  dim3 grid((s.n_qt + kRunTiles - 1) / kRunTiles, n_seg);
  hipLaunchKernelGGL((chunk_attend_kernel<D, BF16>), grid, dim3(256), 0, stream, qk, v, perm, s, o, z);
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
  if (d == 64) {
    return bf16 ? launch_typed<64, true>(qk, v, perm, n_seg, s, o_rounds, z_rounds, stream)
                : launch_typed<64, false>(qk, v, perm, n_seg, s, o_rounds, z_rounds, stream);
  }
  return bf16 ? launch_typed<128, true>(qk, v, perm, n_seg, s, o_rounds, z_rounds, stream)
              : launch_typed<128, false>(qk, v, perm, n_seg, s, o_rounds, z_rounds, stream);
}

}  // namespace rlsh
