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
// tile are contiguous and load as 16-byte coalesced pieces.  Key tiles sit on
// a fixed grid of 64 positions.  A workgroup walks a run of consecutive query
// tiles of 64 positions (one wavefront per 16 queries) and keeps the key tiles
// their windows cover in a ring of R LDS slots (tile t in slot t % R): the
// windows of neighbouring query tiles overlap, so each key tile is read from
// HBM once per run, and the one new tile the next query tile needs is loaded
// into registers while the current one is computed.  Windows spanning more
// than three tiles stream every covered tile through one LDS slot instead.
// Each query keeps an online softmax in the log2 domain.  S^T = K Q^T runs on MFMA (bf16
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

// A lane's query operand: bf16 16x16x32 or float32 16x16x4 B fragments.
template <int D, bool BF16>
struct LocalQOp {
  static constexpr int kQF = BF16 ? D / 32 : D / 4;
  using QFrag = typename std::conditional<BF16, bf16x8, float>::type;
  QFrag f[kQF];
};

// Per-query state of the online softmax and the query operand.
template <int D, bool BF16>
struct LocalQuery {
  static constexpr int kQF = LocalQOp<D, BF16>::kQF;
  LocalQOp<D, BF16> q;
  float m_run, l_run;
  f32x4 oacc[D / 16];
  int qp, wlo, whi;
  bool live;
};

// This lane's query operand for query tile qt (zeros past the sequence).
template <int D, bool BF16>
__device__ __forceinline__ void local_load_q(LocalQOp<D, BF16>& op, const void* __restrict__ q_raw, int L,
                                             size_t row0, int qt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q16 = lane & 15, g = lane >> 4;
  const int qp = qt * kLQTile + 16 * wave + q16;
  const bool live = qp < L;
  if constexpr (BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(q_raw);
#pragma unroll
    for (int kk = 0; kk < LocalQuery<D, BF16>::kQF; ++kk) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (live) raw = *reinterpret_cast<const u32x4*>(q + (row0 + qp) * D + 32 * kk + 8 * g);
      op.f[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  } else {
    const float* q = static_cast<const float*>(q_raw);
#pragma unroll
    for (int kk = 0; kk < LocalQuery<D, BF16>::kQF; ++kk) op.f[kk] = live ? q[(row0 + qp) * D + 4 * kk + g] : 0.0f;
  }
}

// Window and softmax state of this lane's query in tile qt; the operand comes
// from local_load_q.
template <int D, bool BF16>
__device__ __forceinline__ void local_query_init(LocalQuery<D, BF16>& st, const LocalShape& s, int qt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = s.seq_len, m = s.chunk;
  st.qp = qt * kLQTile + 16 * wave + (lane & 15);
  st.live = st.qp < L;
  const int cq = st.live ? st.qp / m : 0;
  st.wlo = max(0, (cq - s.n_before) * m);
  st.whi = st.live ? min(L, (cq + 1 + s.n_after) * m) : 0;
  if (s.causal) st.whi = min(st.whi, st.qp + 1);
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// One key tile of 64 positions starting at kt0, from LDS: scores, window mask,
// online-softmax update and O^T += V^T P^T.
template <int D, bool BF16>
__device__ __forceinline__ void local_tile(LocalQuery<D, BF16>& st, const LocalLds<D, BF16>& t, int kt0,
                                           float scale_log2) {
  using Lds = LocalLds<D, BF16>;
  constexpr int kQF = LocalQuery<D, BF16>::kQF;
  const int lane = threadIdx.x & 63;
  const int q16 = lane & 15, g = lane >> 4;
  // S^T for 4 subtiles of 16 keys: lane holds S[query q16][key 16t + 4g + j].
  f32x4 sc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (BF16) {
#pragma unroll
      for (int kk = 0; kk < kQF; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&t.k[(16 * u + q16) * Lds::kKPitch + 32 * kk + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), st.q.f[kk], acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < kQF; ++kk) {
        const float a = t.k[(16 * u + q16) * Lds::kKPitch + 4 * kk + g];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, st.q.f[kk], acc, 0, 0, 0);
      }
    }
    sc[u] = acc;
  }
  // Window mask on the raw scores; the scale goes into the exponent.
  float tmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kpos = kt0 + 16 * u + 4 * g + j;
      sc[u][j] = (kpos >= st.wlo && kpos < st.whi) ? sc[u][j] : -INFINITY;
      tmax = fmaxf(tmax, sc[u][j]);
    }
  tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
  tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
  const float m_new = fmaxf(st.m_run, tmax);
  const float m_off = (m_new == -INFINITY) ? 0.0f : -m_new * scale_log2;
  const float alpha = (st.m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(st.m_run, scale_log2, m_off));
  float psum = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[u][j], scale_log2, m_off));
      sc[u][j] = p;
      psum += p;
    }
  st.l_run = st.l_run * alpha + psum;
  st.m_run = m_new;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) st.oacc[dt][j] *= alpha;

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
      const uint16_t* vbase = &t.v[(32 * kb + 4 * g + (q16 >> 2)) * Lds::kVPitch + 4 * (q16 & 3)];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const u32x2 lo = lds_read_tr16(vbase + 16 * dt);
        const u32x2 hi = lds_read_tr16(vbase + 16 * Lds::kVPitch + 16 * dt);
        u32x4 a;
        a[0] = lo[0];
        a[1] = lo[1];
        a[2] = hi[0];
        a[3] = hi[1];
        st.oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), bop, st.oacc[dt], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kr = 16 * u + 4 * g + j;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const float a = t.v[kr * Lds::kVPitch + 16 * dt + q16];
          st.oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sc[u][j], st.oacc[dt], 0, 0, 0);
        }
      }
  }
}

template <int D, bool BF16>
__device__ __forceinline__ void local_query_end(const LocalQuery<D, BF16>& st, size_t row0, void* __restrict__ out_raw) {
  const int g = (threadIdx.x & 63) >> 4;
  float lsum = st.l_run;
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);
  if (!st.live) return;
  const float inv = 1.0f / lsum;   // the query's own position is always in its window
  if constexpr (BF16) {
    uint16_t* op = static_cast<uint16_t*>(out_raw) + (row0 + st.qp) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      u32x2 r;
      r[0] = pack_bf16x2(st.oacc[dt][0] * inv, st.oacc[dt][1] * inv);
      r[1] = pack_bf16x2(st.oacc[dt][2] * inv, st.oacc[dt][3] * inv);
      *reinterpret_cast<u32x2*>(op + 16 * dt + 4 * g) = r;
    }
  } else {
    float* op = static_cast<float*>(out_raw) + (row0 + st.qp) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = st.oacc[dt][j] * inv;
      *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g) = r;
    }
  }
}

// Key tiles [a, b) of the fixed 64-position grid that cover the windows of
// query tile qt.
__host__ __device__ inline void local_key_tiles(const LocalShape& s, int qt, int& a, int& b) {
  const int p0 = qt * kLQTile;
  const int p1 = min(p0 + kLQTile, s.seq_len) - 1;
  const int ks_begin = max(0, (p0 / s.chunk - s.n_before) * s.chunk);
  int ks_end = min(s.seq_len, (p1 / s.chunk + 1 + s.n_after) * s.chunk);
  if (s.causal) ks_end = min(ks_end, p1 + 1);
  a = ks_begin / kLKTile;
  b = (ks_end + kLKTile - 1) / kLKTile;
}

// Rows 64t .. 64t + 63 of K and V (clamped to the sequence; rows past it are
// masked by every window) straight into an LDS slot.
template <int D, bool BF16>
__device__ __forceinline__ void local_load_tile(LocalLds<D, BF16>& t, const void* __restrict__ k_raw,
                                                const void* __restrict__ v_raw, size_t row0, int L, int tile) {
  using Lds = LocalLds<D, BF16>;
  constexpr int kPieces = BF16 ? D / 8 : D / 4;
  for (int u = threadIdx.x; u < kLKTile * kPieces; u += 256) {
    const int row = u / kPieces, pc = u % kPieces;
    const int pos = min(tile * kLKTile + row, L - 1);
    if constexpr (BF16) {
      const size_t src = (row0 + pos) * D + 8 * pc;
      *reinterpret_cast<u32x4*>(&t.k[row * Lds::kKPitch + 8 * pc]) =
          *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(k_raw) + src);
      *reinterpret_cast<u32x4*>(&t.v[row * Lds::kVPitch + 8 * pc]) =
          *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(v_raw) + src);
    } else {
      const size_t src = (row0 + pos) * D + 4 * pc;
      *reinterpret_cast<f32x4*>(&t.k[row * Lds::kKPitch + 4 * pc]) =
          *reinterpret_cast<const f32x4*>(static_cast<const float*>(k_raw) + src);
      *reinterpret_cast<f32x4*>(&t.v[row * Lds::kVPitch + 4 * pc]) =
          *reinterpret_cast<const f32x4*>(static_cast<const float*>(v_raw) + src);
    }
  }
}

// bf16 key tile in flight in registers: one 16-byte piece of K and of V per
// thread and step.
template <int D>
struct LocalTileRegs {
  static constexpr int kPer = kLKTile * (D / 8) / 256;
  u32x4 k[kPer], v[kPer];
};

template <int D>
__device__ __forceinline__ void local_gather_regs(LocalTileRegs<D>& r, const uint16_t* __restrict__ kp,
                                                  const uint16_t* __restrict__ vp, size_t row0, int L, int tile) {
#pragma unroll
  for (int i = 0; i < LocalTileRegs<D>::kPer; ++i) {
    const int u = threadIdx.x + 256 * i;
    const int row = u / (D / 8), pc = u % (D / 8);
    const size_t src = (row0 + min(tile * kLKTile + row, L - 1)) * D + 8 * pc;
    r.k[i] = *reinterpret_cast<const u32x4*>(kp + src);
    r.v[i] = *reinterpret_cast<const u32x4*>(vp + src);
  }
}

template <int D>
__device__ __forceinline__ void local_store_regs(const LocalTileRegs<D>& r, LocalLds<D, true>& t) {
  using Lds = LocalLds<D, true>;
#pragma unroll
  for (int i = 0; i < LocalTileRegs<D>::kPer; ++i) {
    const int u = threadIdx.x + 256 * i;
    const int row = u / (D / 8), pc = u % (D / 8);
    *reinterpret_cast<u32x4*>(&t.k[row * Lds::kKPitch + 8 * pc]) = r.k[i];
    *reinterpret_cast<u32x4*>(&t.v[row * Lds::kVPitch + 8 * pc]) = r.v[i];
  }
}

constexpr int kRingRun = 16;   // query tiles per workgroup on the ring path

// Ring path: every query tile's windows fit in R key tiles.
template <int D, bool BF16, int R>
__global__ __launch_bounds__(256) void local_ring_kernel(const void* __restrict__ q_raw, const void* __restrict__ k_raw,
                                                         const void* __restrict__ v_raw, LocalShape s,
                                                         void* __restrict__ out_raw) {
  __shared__ LocalLds<D, BF16> ring[R];
  const int L = s.seq_len;
  const size_t row0 = static_cast<size_t>(blockIdx.y) * L;
  const int qt_begin = blockIdx.x * kRingRun;
  const int qt_end = min(s.n_qt, qt_begin + kRingRun);
  int a, b;
  local_key_tiles(s, qt_begin, a, b);
  for (int t = a; t < b; ++t) local_load_tile<D, BF16>(ring[t % R], k_raw, v_raw, row0, L, t);
  int loaded = b;   // tiles below `loaded` have been brought in (the last R of them are resident)
  __syncthreads();
  for (int qt = qt_begin; qt < qt_end; ++qt) {
    local_key_tiles(s, qt, a, b);
    int na = 0, nb = loaded;
    if (qt + 1 < qt_end) local_key_tiles(s, qt + 1, na, nb);
    // the next query tile's single new key tile, into registers during this one
    const bool one_new = BF16 && nb == loaded + 1;
    LocalTileRegs<D> pre;
    if constexpr (BF16) {
      if (one_new)
        local_gather_regs<D>(pre, static_cast<const uint16_t*>(k_raw), static_cast<const uint16_t*>(v_raw), row0, L,
                             loaded);
    }
    LocalQuery<D, BF16> st;
    local_load_q<D, BF16>(st.q, q_raw, L, row0, qt);
    local_query_init<D, BF16>(st, s, qt);
    for (int t = a; t < b; ++t) local_tile<D, BF16>(st, ring[t % R], t * kLKTile, s.scale_log2);
    local_query_end<D, BF16>(st, row0, out_raw);
    if (nb > loaded) {
      __syncthreads();   // every wavefront is done with the slots the new tiles take
      if constexpr (BF16) {
        if (one_new) local_store_regs<D>(pre, ring[loaded % R]);
      }
      if (!one_new)
        for (int t = loaded; t < nb; ++t) local_load_tile<D, BF16>(ring[t % R], k_raw, v_raw, row0, L, t);
      loaded = nb;
      __syncthreads();
    }
  }
}

// General path: windows wider than the ring; every covered key tile streams
// through one LDS slot.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void local_stream_kernel(const void* __restrict__ q_raw,
                                                           const void* __restrict__ k_raw,
                                                           const void* __restrict__ v_raw, LocalShape s,
                                                           void* __restrict__ out_raw) {
  __shared__ LocalLds<D, BF16> sh;
  const int L = s.seq_len;
  const size_t row0 = static_cast<size_t>(blockIdx.y) * L;
  const int qt_begin = blockIdx.x * kLRunTiles;
  const int qt_end = min(s.n_qt, qt_begin + kLRunTiles);
  for (int qt = qt_begin; qt < qt_end; ++qt) {
    int a, b;
    local_key_tiles(s, qt, a, b);
    LocalQuery<D, BF16> st;
    local_load_q<D, BF16>(st.q, q_raw, L, row0, qt);
    local_query_init<D, BF16>(st, s, qt);
    for (int t = a; t < b; ++t) {
      __syncthreads();   // earlier readers of the LDS tile are done
      local_load_tile<D, BF16>(sh, k_raw, v_raw, row0, L, t);
      __syncthreads();
      local_tile<D, BF16>(st, sh, t * kLKTile, s.scale_log2);
    }
    local_query_end<D, BF16>(st, row0, out_raw);
  }
}

template <int D, bool BF16>
hipError_t launch_local_typed(const void* q, const void* k, const void* v, int bh, const LocalShape& s, void* out,
                              hipStream_t stream) {
  // widest key-tile span of any query tile
  int span = 0;
  for (int qt = 0; qt < s.n_qt; ++qt) {
    int a, b;
    local_key_tiles(s, qt, a, b);
    span = std::max(span, b - a);
  }
  const dim3 ring_grid((s.n_qt + kRingRun - 1) / kRingRun, bh);
  constexpr bool kThreeFit = sizeof(LocalLds<D, BF16>) * 3 <= 160 * 1024;   // LDS per workgroup
  if (span <= 2) {
    hipLaunchKernelGGL((local_ring_kernel<D, BF16, 2>), ring_grid, dim3(256), 0, stream, q, k, v, s, out);
    return hipGetLastError();
  }
  if constexpr (kThreeFit) {
    if (span <= 3) {
      hipLaunchKernelGGL((local_ring_kernel<D, BF16, 3>), ring_grid, dim3(256), 0, stream, q, k, v, s, out);
      return hipGetLastError();
    }
  }
  dim3 grid((s.n_qt + kLRunTiles - 1) / kLRunTiles, bh);
  hipLaunchKernelGGL((local_stream_kernel<D, BF16>), grid, dim3(256), 0, stream, q, k, v, s, out);
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
