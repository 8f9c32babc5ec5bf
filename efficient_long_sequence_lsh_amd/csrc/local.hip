// Local (sliding-chunk) self-attention.
//
// "The Reformer - Pushing the limits of language modeling" (summary page),
// Approach / What changed and Takeaways: besides LSH attention the model uses
// local self-attention, where the sequence is cut into chunks of length l_c
// and each chunk attends to itself plus an overlap of preceding and following
// chunks, so that every position keeps its immediate neighbours.
//
// Readings taken here (the page gives no more): queries, keys and values are
// separate tensors (q may alias k); query i in chunk c = i / m' attends to the
// keys of chunks c - n_before .. c + n_after that exist (no wrap-around),
// m' = min(l_c, L), L a multiple of m'; causal keeps keys j <= i; there is no
// self-mask (a position may attend to itself, so no query is ever without a
// key); score q_i . k_j / sqrt(d), one softmax over the window.
//
// Design for gfx950: positions are not permuted, so K and V rows of a key
// tile are contiguous and load as 16-byte coalesced pieces.  A workgroup owns
// 4 consecutive query tiles of 64 positions (one wavefront per 16 queries);
// for each it streams the key tiles its windows cover through LDS and keeps an
// online softmax in the log2 domain.  S^T = K Q^T runs on MFMA (bf16
// 16x16x32, or float32 16x16x4), so each lane owns one query -- the B-operand
// layout of O^T = V^T P^T.  The bf16 V tile is stored row-major and read with
// the transposing LDS read ds_read_b64_tr_b16.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace rlsh {

namespace {

constexpr int kLQTile = 64;     // queries per tile (4 wavefronts x 16)
constexpr int kLKTile = 64;     // keys per LDS tile
constexpr int kLRunTiles = 4;   // query tiles per workgroup

struct LocalShape {
  int seq_len;
  int chunk;      // m' = min(l_c, L)
  int n_before;
  int n_after;
  int causal;
  int n_qt;       // query tiles per (batch, head)
  float scale_log2;
};

template <int D, bool BF16>
struct LocalLds;

template <int D>
struct alignas(16) LocalLds<D, true> {
  static constexpr int kKPitch = D + 8;    // 16-byte pad: conflict-free 16-byte row reads
  static constexpr int kVPitch = D + 16;   // conflict-free transposing reads
  uint16_t k[kLKTile * kKPitch];
  uint16_t v[kLKTile * kVPitch];
};

template <int D>
struct alignas(16) LocalLds<D, false> {
  static constexpr int kKPitch = D + 4;
  static constexpr int kVPitch = D + 4;
  float k[kLKTile * kKPitch];
  float v[kLKTile * kVPitch];
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void local_attend_kernel(const void* __restrict__ q_raw,
                                                           const void* __restrict__ k_raw,
                                                           const void* __restrict__ v_raw, LocalShape s,
                                                           void* __restrict__ out_raw) {
  using Lds = LocalLds<D, BF16>;
  __shared__ Lds sh;
  const int bh = blockIdx.y;
  const int L = s.seq_len;
  const int m = s.chunk;
  const size_t row0 = static_cast<size_t>(bh) * L;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q16 = lane & 15;
  const int g = lane >> 4;
  const int qt_begin = blockIdx.x * kLRunTiles;
  const int qt_end = min(s.n_qt, qt_begin + kLRunTiles);

  for (int qt = qt_begin; qt < qt_end; ++qt) {
    const int p0 = qt * kLQTile;
    const int qp = p0 + 16 * wave + q16;     // this lane's query position
    const bool qlive = qp < L;
    const int cq = qlive ? qp / m : 0;
    const int wlo = max(0, (cq - s.n_before) * m);
    int whi = qlive ? min(L, (cq + 1 + s.n_after) * m) : 0;
    if (s.causal) whi = min(whi, qp + 1);
    // Key range covering the windows of the whole query tile.
    const int p1 = min(p0 + kLQTile, L) - 1;
    const int ks_begin = max(0, (p0 / m - s.n_before) * m);
    int ks_end = min(L, (p1 / m + 1 + s.n_after) * m);
    if (s.causal) ks_end = min(ks_end, p1 + 1);

    constexpr int kQF = BF16 ? D / 32 : D / 4;
    using QFrag = typename std::conditional<BF16, bf16x8, float>::type;
    QFrag qf[kQF];
    if constexpr (BF16) {
      const uint16_t* q = static_cast<const uint16_t*>(q_raw);
#pragma unroll
      for (int kk = 0; kk < kQF; ++kk) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qlive) raw = *reinterpret_cast<const u32x4*>(q + (row0 + qp) * D + 32 * kk + 8 * g);
        qf[kk] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
      const float* q = static_cast<const float*>(q_raw);
#pragma unroll
      for (int kk = 0; kk < kQF; ++kk) qf[kk] = qlive ? q[(row0 + qp) * D + 4 * kk + g] : 0.0f;
    }

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x4 oacc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int kt0 = ks_begin; kt0 < ks_end; kt0 += kLKTile) {
      __syncthreads();   // earlier readers of the LDS tile are done
      if constexpr (BF16) {
        const uint16_t* kp = static_cast<const uint16_t*>(k_raw);
        const uint16_t* vp = static_cast<const uint16_t*>(v_raw);
        constexpr int kPieces = D / 8;
        for (int u = threadIdx.x; u < kLKTile * kPieces; u += 256) {
          const int row = u / kPieces, pc = u % kPieces;
          const int pos = min(kt0 + row, ks_end - 1);   // rows past the range are masked below
          const size_t src = (row0 + pos) * D + 8 * pc;
          *reinterpret_cast<u32x4*>(&sh.k[row * Lds::kKPitch + 8 * pc]) = *reinterpret_cast<const u32x4*>(kp + src);
          *reinterpret_cast<u32x4*>(&sh.v[row * Lds::kVPitch + 8 * pc]) = *reinterpret_cast<const u32x4*>(vp + src);
        }
      } else {
        const float* kp = static_cast<const float*>(k_raw);
        const float* vp = static_cast<const float*>(v_raw);
        constexpr int kPieces = D / 4;
        for (int u = threadIdx.x; u < kLKTile * kPieces; u += 256) {
          const int row = u / kPieces, pc = u % kPieces;
          const int pos = min(kt0 + row, ks_end - 1);
          const size_t src = (row0 + pos) * D + 4 * pc;
          *reinterpret_cast<f32x4*>(&sh.k[row * Lds::kKPitch + 4 * pc]) = *reinterpret_cast<const f32x4*>(kp + src);
          *reinterpret_cast<f32x4*>(&sh.v[row * Lds::kVPitch + 4 * pc]) = *reinterpret_cast<const f32x4*>(vp + src);
        }
      }
      __syncthreads();

      // S^T for 4 subtiles of 16 keys: lane holds S[query q16][key 16t + 4g + j].
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
      // Window mask on the raw scores; the scale goes into the exponent.
      float tmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kpos = kt0 + 16 * t + 4 * g + j;
          sc[t][j] = (kpos >= wlo && kpos < whi) ? sc[t][j] : -INFINITY;
          tmax = fmaxf(tmax, sc[t][j]);
        }
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_off = (m_new == -INFINITY) ? 0.0f : -m_new * s.scale_log2;
      const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(m_run, s.scale_log2, m_off));
      float psum = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[t][j], s.scale_log2, m_off));
          sc[t][j] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) oacc[dt][j] *= alpha;

      if constexpr (BF16) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 pb;
          pb[0] = pack_bf16x2(sc[2 * kb][0], sc[2 * kb][1]);
          pb[1] = pack_bf16x2(sc[2 * kb][2], sc[2 * kb][3]);
          pb[2] = pack_bf16x2(sc[2 * kb + 1][0], sc[2 * kb + 1][1]);
          pb[3] = pack_bf16x2(sc[2 * kb + 1][2], sc[2 * kb + 1][3]);
          const bf16x8 bop = __builtin_bit_cast(bf16x8, pb);
          // V^T operand: lane 16g + i needs feature i of keys 32kb + 4g + {0..3}
          // and 32kb + 16 + 4g + {0..3}; lane 16g + 4k + q points at key row
          // (.. + k), features 16dt + 4q .. +3.
          const uint16_t* vbase = &sh.v[(32 * kb + 4 * g + (q16 >> 2)) * Lds::kVPitch + 4 * (q16 & 3)];
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const u32x2 lo = lds_read_tr16(vbase + 16 * dt);
            const u32x2 hi = lds_read_tr16(vbase + 16 * Lds::kVPitch + 16 * dt);
            u32x4 a;
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

    float lsum = l_run;
    lsum += shfl_xor_f(lsum, 16);
    lsum += shfl_xor_f(lsum, 32);
    if (qlive) {
      const float inv = 1.0f / lsum;   // the query's own position is always in its window
      if constexpr (BF16) {
        uint16_t* op = static_cast<uint16_t*>(out_raw) + (row0 + qp) * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          u32x2 r;
          r[0] = pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv);
          r[1] = pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv);
          *reinterpret_cast<u32x2*>(op + 16 * dt + 4 * g) = r;
        }
      } else {
        float* op = static_cast<float*>(out_raw) + (row0 + qp) * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          f32x4 r;
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = oacc[dt][j] * inv;
          *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g) = r;
        }
      }
    }
  }
}

template <int D, bool BF16>
hipError_t launch_local_typed(const void* q, const void* k, const void* v, int bh, const LocalShape& s, void* out,
                              hipStream_t stream) {
  dim3 grid((s.n_qt + kLRunTiles - 1) / kLRunTiles, bh);
  hipLaunchKernelGGL((local_attend_kernel<D, BF16>), grid, dim3(256), 0, stream, q, k, v, s, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_local_attend(const void* q, const void* k, const void* v, bool bf16, int bh, int seq_len, int d,
                               int chunk_len, int n_before, int n_after, bool causal, void* out, hipStream_t stream) {
  LocalShape s{};
  s.seq_len = seq_len;
  s.chunk = std::min(chunk_len, seq_len);
  s.n_before = n_before;
  s.n_after = n_after;
  s.causal = causal ? 1 : 0;
  s.n_qt = (seq_len + kLQTile - 1) / kLQTile;
  s.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
  if (d == 64)
    return bf16 ? launch_local_typed<64, true>(q, k, v, bh, s, out, stream)
                : launch_local_typed<64, false>(q, k, v, bh, s, out, stream);
  return bf16 ? launch_local_typed<128, true>(q, k, v, bh, s, out, stream)
              : launch_local_typed<128, false>(q, k, v, bh, s, out, stream);
}

}  // namespace rlsh
