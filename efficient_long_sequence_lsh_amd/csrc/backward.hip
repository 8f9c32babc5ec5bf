// Gradients of the LSH attention forward with respect to the shared vectors
// qk and the values v, for a given sorted order (the hash is held fixed: bucket
// ids are piecewise constant in the inputs).
//
// "Reformer: The Efficient Transformer" (research summary), Key points: the
// sorted positions form chunks of m whose queries see their own chunk's and the
// preceding chunk's keys (LSH attention bullet); a token attends to itself only when it has no other
// target (Shared-QK bullet); several rounds are combined (Number of hash
// rounds bullet; combined here with logsumexp weights).  With Z_i the
// logsumexp of the scores of all (round, key) pairs query i sees, the forward
// is out_i = sum_{rho, j} P_rho,ij v_j with P = exp(s_ij - Z_i), so with
// D_i = dout_i . out_i:
//   dv_j  += sum_{rho, i} P_rho,ij dout_i          (+ dout_j for self-fallback rows)
//   dS    =  P (dout_i . v_j - D_i)
//   dqk_i += sum dS_ij qk_j / sqrt(d)   (query role)
//   dqk_j += sum dS_ij qk_i / sqrt(d)   (key role)
//
// Design for gfx950 (chunks of 64 slots).  bf16 inputs: S and dP on the bf16
// MFMA 16x16x32 (products of bf16 inputs are exact in float32), P and dS
// rounded to bf16 for the gradient contractions, whose transposed operands come
// from the gfx950 transposing LDS read; float32 inputs: every contraction on
// the float32 MFMA 16x16x4 with rows widened in LDS.
//   z pass      per round, per query chunk (bf16: runs of chunks per
//               workgroup): the query's log2-domain normaliser over its
//               window (chunks c-1 and c), written per position.
//   stats       per position: Z (log2 domain, over rounds) and D.
//   key pass    per round, per key chunk c: its keys are seen by the queries
//               of chunks c and c+1; each wavefront owns 16 keys, streams the
//               128 queries through LDS, and accumulates dv^T and dk^T
//               (feature x key tiles) in registers; then adds them to the rows
//               of its keys (round 0 writes them, with dout added to dv on
//               self-fallback rows, so no separate initialisation pass is
//               needed).
//   query pass  per round, per query chunk c: keys of chunks c-1 and c; each
//               wavefront owns 16 queries and accumulates dq^T.
// float32 inputs run the two passes as separate kernels; bf16 inputs run both
// in one kernel over runs of consecutive chunks (below), which gathers every
// row once per round instead of three times.  Within a round every position
// is one key of one key chunk and one query of one query chunk, so each row
// has a single writing workgroup; rounds run one after another on the stream,
// so the read-add-write of the float32 gradient rows never races.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>
#include <cmath>

namespace rlsh {

namespace {

constexpr int kBT = 64;          // slots per chunk and per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

struct BwdShape {
  int seq_len;
  int n_rounds;
  int n_chunks;    // seq_len / 64
  int causal;
  float scale;     // 1 / sqrt(d)
  float scale_log2;
};

template <int D>
struct alignas(16) BwdTile {
  static constexpr int kPitch = D + 4;   // floats per row: conflict-free column reads
  float a[kBT * kPitch];                 // q rows (key pass) or k rows (query pass)
  float b[kBT * kPitch];                 // dout rows (key pass) or v rows (query pass)
  int pos[kBT];
  int slot[kBT];
  float z2[kBT];                         // key pass: Z of the queries (log2 domain)
  float dd[kBT];                         // key pass: D of the queries
};

// Rows of one 64-slot chunk, gathered through perm and widened to float32.
template <int D, bool BF16>
__device__ __forceinline__ void stage_rows(float* dst, const void* src_raw, const int32_t* perm, int c, size_t row0) {
  constexpr int kP = BwdTile<D>::kPitch;
  if constexpr (BF16) {
    const uint16_t* src = static_cast<const uint16_t*>(src_raw);
    for (int u = threadIdx.x; u < kBT * (D / 8); u += blockDim.x) {
      const int row = u / (D / 8), pc = u % (D / 8);
      const u32x4 raw = *reinterpret_cast<const u32x4*>(src + (row0 + perm[c * kBT + row]) * D + 8 * pc);
      float* o = dst + row * kP + 8 * pc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = __uint_as_float(raw[e] << 16);
        o[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
      }
    }
  } else {
    const float* src = static_cast<const float*>(src_raw);
    for (int u = threadIdx.x; u < kBT * (D / 4); u += blockDim.x) {
      const int row = u / (D / 4), pc = u % (D / 4);
      *reinterpret_cast<f32x4*>(dst + row * kP + 4 * pc) =
          *reinterpret_cast<const f32x4*>(src + (row0 + perm[c * kBT + row]) * D + 4 * pc);
    }
  }
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

// ------------------------------------------------------------- z pass ----
// grid (n_chunks, bh * n_rounds); wavefront w owns queries 16w..16w+15 of the
// chunk.  z2 = log2 sum_j 2^(s_ij * scale_log2) over the valid window keys
// (-inf when there is none).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_z_kernel(const void* __restrict__ qk, const int32_t* __restrict__ perm_all,
                                                    BwdShape s, float* __restrict__ z2_rounds) {
  __shared__ BwdTile<D> sh;
  constexpr int kP = BwdTile<D>::kPitch;
  const int c = blockIdx.x, seg = blockIdx.y;
  const int bh = seg / s.n_rounds;
  const int L = s.seq_len;
  const int32_t* perm = perm_all + static_cast<size_t>(seg) * L;
  const size_t row0 = static_cast<size_t>(bh) * L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int qslot = c * kBT + 16 * wave + c16;
  const int qpos = perm[qslot];
  // B operand of S^T = K Q^T: lane (g, c16) holds q[c16][4kk + g].
  float qreg[D / 4];
#pragma unroll
  for (int kk = 0; kk < D / 4; ++kk) qreg[kk] = load_elem<BF16>(qk, (row0 + qpos) * D + 4 * kk + g);
  float mrun = -INFINITY, lrun = 0.0f;
  for (int h = (c > 0 ? 0 : 1); h < 2; ++h) {
    const int kc = c - 1 + h;
    __syncthreads();
    stage_rows<D, BF16>(sh.a, qk, perm, kc, row0);
    if (threadIdx.x < kBT) {
      sh.pos[threadIdx.x] = perm[kc * kBT + threadIdx.x];
      sh.slot[threadIdx.x] = kc * kBT + threadIdx.x;
    }
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.a[(16 * kt + c16) * kP + 4 * kk + g], qreg[kk], acc, 0, 0, 0);
      // lane holds S^T[key 16kt + 4g + j][query c16]
      float tmax = -INFINITY;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kr = 16 * kt + 4 * g + j;
        bool ok = sh.slot[kr] != qslot;
        if (s.causal) ok = ok && sh.pos[kr] < qpos;
        v[j] = ok ? acc[j] * s.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, v[j]);
      }
      const float mnew = fmaxf(mrun, tmax);
      if (mnew != -INFINITY) {
        float add = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) add += exp2f(v[j] - mnew);
        lrun = lrun * exp2f(mrun - mnew) + add;
        mrun = mnew;
      }
    }
  }
  // Merge the four lanes (g = 0..3) that share query c16.
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const float om = shfl_xor_f(mrun, off), ol = shfl_xor_f(lrun, off);
    const float mnew = fmaxf(mrun, om);
    if (mnew != -INFINITY) {
      lrun = lrun * exp2f(mrun - mnew) + ol * exp2f(om - mnew);
      mrun = mnew;
    }
  }
  if (g == 0) z2_rounds[static_cast<size_t>(seg) * L + qpos] = (mrun == -INFINITY) ? -INFINITY : mrun + log2f(lrun);
}

// -------------------------------------------------------------- stats ----
// D/8 lanes per position (8 features each): Z (log2 domain) over rounds and
// D = dout . out.  With the forward's log normaliser (lse, natural log) Z is
// that value times log2(e) and the per-round values are not read.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const float* __restrict__ z2_rounds, const float* __restrict__ lse,
                                                        const void* __restrict__ out, const void* __restrict__ dout,
                                                        int n_rows, int seq_len, int n_rounds, float* __restrict__ z2,
                                                        float* __restrict__ dd) {
  constexpr int kT = D / 8;
  const int row = (blockIdx.x * blockDim.x + threadIdx.x) / kT;
  const int sub = threadIdx.x % kT;
  const bool live = row < n_rows;
  const size_t r = live ? static_cast<size_t>(row) : 0;
  float acc = 0.0f;
  if constexpr (BF16) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(out) + r * D + 8 * sub);
    const u32x4 b = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(dout) + r * D + 8 * sub);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), acc);
      acc = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(b[e] & 0xffff0000u), acc);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(out) + r * D + 8 * sub + 4 * h);
      const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(dout) + r * D + 8 * sub + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(a[e], b[e], acc);
    }
  }
#pragma unroll
  for (int off = 1; off < kT; off <<= 1) acc += __shfl_xor(acc, off, kT);
  if (!live || sub != 0) return;
  dd[row] = acc;
  if (lse != nullptr) {
    z2[row] = lse[row] * kLog2e;   // -inf stays -inf
    return;
  }
  const int bh = row / seq_len, pos = row - bh * seq_len;
  const float* zr = z2_rounds + static_cast<size_t>(bh) * n_rounds * seq_len + pos;
  float m = -INFINITY;
  for (int k = 0; k < n_rounds; ++k) m = fmaxf(m, zr[static_cast<size_t>(k) * seq_len]);
  float zz = -INFINITY;
  if (m != -INFINITY) {
    float sum = 0.0f;
    for (int k = 0; k < n_rounds; ++k) sum += exp2f(zr[static_cast<size_t>(k) * seq_len] - m);
    zz = m + log2f(sum);
  }
  z2[row] = zz;
}

// Add (or, in round 0, write) the key-side gradients of one key: the lane
// holds features 16dt + 4g + j of key row kpos.  Round 0 also adds dout to dv
// on a self-fallback row (out = v there).
template <int D, bool BF16>
__device__ __forceinline__ void store_key_grads(const f32x4 (&dvt)[D / 16], const f32x4 (&dkt)[D / 16], size_t row0,
                                                int kpos, int g, int round, const float* __restrict__ z2,
                                                const void* __restrict__ dout, float scale, float* __restrict__ dqk,
                                                float* __restrict__ dv) {
  float* dvr = dv + (row0 + kpos) * D;
  float* dkr = dqk + (row0 + kpos) * D;
  const bool fallback = round == 0 && z2[row0 + kpos] == -INFINITY;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    f32x4 a = dvt[dt];
    f32x4 b;
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = dkt[dt][j] * scale;
    if (round == 0) {
      if (fallback) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] += load_elem<BF16>(dout, (row0 + kpos) * D + 16 * dt + 4 * g + j);
      }
    } else {
      const f32x4 pa = *reinterpret_cast<const f32x4*>(dvr + 16 * dt + 4 * g);
      const f32x4 pb = *reinterpret_cast<const f32x4*>(dkr + 16 * dt + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] += pa[j];
        b[j] += pb[j];
      }
    }
    *reinterpret_cast<f32x4*>(dvr + 16 * dt + 4 * g) = a;
    *reinterpret_cast<f32x4*>(dkr + 16 * dt + 4 * g) = b;
  }
}

// ------------------------------------------------------------ key pass ----
// grid (n_chunks, bh) for one round.  Wavefront w owns keys 16w..16w+15 of key
// chunk c; the queries are chunks c (own) and c+1 (next).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_key_kernel(const void* __restrict__ qk, const void* __restrict__ vv,
                                                      const void* __restrict__ dout, const int32_t* __restrict__ perm_all,
                                                      BwdShape s, int round, const float* __restrict__ z2,
                                                      const float* __restrict__ dd, float* __restrict__ dqk,
                                                      float* __restrict__ dv) {
  __shared__ BwdTile<D> sh;
  constexpr int kP = BwdTile<D>::kPitch;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int L = s.seq_len;
  const int32_t* perm = perm_all + (static_cast<size_t>(bh) * s.n_rounds + round) * L;
  const size_t row0 = static_cast<size_t>(bh) * L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int kslot = c * kBT + 16 * wave + c16;   // this lane's key column
  const int kpos = perm[kslot];
  // B operands (4 features x 16 keys): lane (g, c16) holds row c16 at feature 4kk + g.
  float kreg[D / 4], vreg[D / 4];
#pragma unroll
  for (int kk = 0; kk < D / 4; ++kk) {
    kreg[kk] = load_elem<BF16>(qk, (row0 + kpos) * D + 4 * kk + g);
    vreg[kk] = load_elem<BF16>(vv, (row0 + kpos) * D + 4 * kk + g);
  }
  f32x4 dvt[D / 16], dkt[D / 16];   // (feature 16dt + 4g + j, key c16)
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    dvt[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    dkt[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const int h_end = (c + 1 < s.n_chunks) ? 2 : 1;
  for (int h = 0; h < h_end; ++h) {
    const int qc = c + h;
    __syncthreads();
    stage_rows<D, BF16>(sh.a, qk, perm, qc, row0);
    stage_rows<D, BF16>(sh.b, dout, perm, qc, row0);
    if (threadIdx.x < kBT) {
      const int p = perm[qc * kBT + threadIdx.x];
      sh.pos[threadIdx.x] = p;
      sh.slot[threadIdx.x] = qc * kBT + threadIdx.x;
      sh.z2[threadIdx.x] = z2[row0 + p];
      sh.dd[threadIdx.x] = dd[row0 + p];
    }
    __syncthreads();
#pragma unroll 1
    for (int qt = 0; qt < 4; ++qt) {
      // S and dP (16 queries x 16 keys): A = q / dout rows (lane (g, c16):
      // row c16, feature 4kk + g), B = k / v in registers.
      f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f}, pacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.a[(16 * qt + c16) * kP + 4 * kk + g], kreg[kk], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.b[(16 * qt + c16) * kP + 4 * kk + g], vreg[kk], pacc, 0, 0, 0);
      }
      // lane holds (query 16qt + 4g + j, key c16)
      float p[4], ds[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qr = 16 * qt + 4 * g + j;
        bool ok = sh.slot[qr] != kslot;
        if (s.causal) ok = ok && kpos < sh.pos[qr];
        const float zq = sh.z2[qr];
        p[j] = (ok && zq != -INFINITY) ? exp2f(fmaf(sacc[j], s.scale_log2, -zq)) : 0.0f;
        ds[j] = p[j] * (pacc[j] - sh.dd[qr]);
      }
      // dv^T += dout^T P, dk^T += q^T dS: MFMA j takes the queries 4g + j as
      // its k index; A = (feature 16dt + c16, query 4g + j).
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qr = 16 * qt + 4 * g + j;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          dvt[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.b[qr * kP + 16 * dt + c16], p[j], dvt[dt], 0, 0, 0);
          dkt[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.a[qr * kP + 16 * dt + c16], ds[j], dkt[dt], 0, 0, 0);
        }
      }
    }
  }
  store_key_grads<D, BF16>(dvt, dkt, row0, kpos, g, round, z2, dout, s.scale, dqk, dv);
}

// ---------------------------------------------------------- query pass ----
// grid (n_chunks, bh) for one round.  Wavefront w owns queries 16w..16w+15 of
// query chunk c; the keys are chunks c-1 (if any) and c.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_query_kernel(const void* __restrict__ qk, const void* __restrict__ vv,
                                                        const void* __restrict__ dout,
                                                        const int32_t* __restrict__ perm_all, BwdShape s, int round,
                                                        const float* __restrict__ z2, const float* __restrict__ dd,
                                                        float* __restrict__ dqk) {
  __shared__ BwdTile<D> sh;
  constexpr int kP = BwdTile<D>::kPitch;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int L = s.seq_len;
  const int32_t* perm = perm_all + (static_cast<size_t>(bh) * s.n_rounds + round) * L;
  const size_t row0 = static_cast<size_t>(bh) * L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int qslot = c * kBT + 16 * wave + c16;   // this lane's query column
  const int qpos = perm[qslot];
  const float zq = z2[row0 + qpos];
  const float dq = dd[row0 + qpos];
  float qreg[D / 4], oreg[D / 4];   // B operands: q and dout of query c16 at feature 4kk + g
#pragma unroll
  for (int kk = 0; kk < D / 4; ++kk) {
    qreg[kk] = load_elem<BF16>(qk, (row0 + qpos) * D + 4 * kk + g);
    oreg[kk] = load_elem<BF16>(dout, (row0 + qpos) * D + 4 * kk + g);
  }
  f32x4 dqt[D / 16];   // (feature 16dt + 4g + j, query c16)
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dqt[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int h = (c > 0 ? 0 : 1); h < 2; ++h) {
    const int kc = c - 1 + h;
    __syncthreads();
    stage_rows<D, BF16>(sh.a, qk, perm, kc, row0);
    stage_rows<D, BF16>(sh.b, vv, perm, kc, row0);
    if (threadIdx.x < kBT) {
      sh.pos[threadIdx.x] = perm[kc * kBT + threadIdx.x];
      sh.slot[threadIdx.x] = kc * kBT + threadIdx.x;
    }
    __syncthreads();
#pragma unroll 1
    for (int kt = 0; kt < 4; ++kt) {
      // S^T and dP^T (16 keys x 16 queries): A = k / v rows from LDS.
      f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f}, pacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.a[(16 * kt + c16) * kP + 4 * kk + g], qreg[kk], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.b[(16 * kt + c16) * kP + 4 * kk + g], oreg[kk], pacc, 0, 0, 0);
      }
      // lane holds (key 16kt + 4g + j, query c16)
      float ds[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kr = 16 * kt + 4 * g + j;
        bool ok = sh.slot[kr] != qslot;
        if (s.causal) ok = ok && sh.pos[kr] < qpos;
        const float p = (ok && zq != -INFINITY) ? exp2f(fmaf(sacc[j], s.scale_log2, -zq)) : 0.0f;
        ds[j] = p * (pacc[j] - dq);
      }
      // dq^T += k^T dS^T: MFMA j takes keys 4g + j as its k index.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kr = 16 * kt + 4 * g + j;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          dqt[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.a[kr * kP + 16 * dt + c16], ds[j], dqt[dt], 0, 0, 0);
      }
    }
  }
  float* dqr = dqk + (row0 + qpos) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    f32x4 a = *reinterpret_cast<const f32x4*>(dqr + 16 * dt + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = fmaf(dqt[dt][j], s.scale, a[j]);
    *reinterpret_cast<f32x4*>(dqr + 16 * dt + 4 * g) = a;
  }
}

// ------------------------------------------------- bf16 MFMA variants ----
template <int D>
struct alignas(16) BwdTile16 {
  static constexpr int kPitch = D + 16;   // bf16 per row: conflict-free transposing reads
  uint16_t a[kBT * kPitch];               // q rows (key pass) or k rows (z and query passes)
  uint16_t b[kBT * kPitch];               // dout rows (key pass) or v rows (query pass)
  int pos[kBT];
  int slot[kBT];
  float z2[kBT];
  float dd[kBT];
};

template <int D>
__device__ __forceinline__ void stage_rows16(uint16_t* dst, const uint16_t* __restrict__ src, const int32_t* perm,
                                             int c, size_t row0) {
  constexpr int kP = BwdTile16<D>::kPitch;
  for (int u = threadIdx.x; u < kBT * (D / 8); u += blockDim.x) {
    const int row = u / (D / 8), pc = u % (D / 8);
    *reinterpret_cast<u32x4*>(dst + row * kP + 8 * pc) =
        *reinterpret_cast<const u32x4*>(src + (row0 + perm[c * kBT + row]) * D + 8 * pc);
  }
}

template <int D>
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* rowp, int kk, int g) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(rowp + 32 * kk + 8 * g));
}

// 16 rows x 16 rows of dot products over d features: A rows from LDS, B rows in registers.
template <int D>
__device__ __forceinline__ f32x4 dot_tile16(const uint16_t* arow, const bf16x8 (&b)[D / 32], int g) {
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag<D>(arow, kk, g), b[kk], acc, 0, 0, 0);
  return acc;
}

// As dot_tile16, with the B rows read from LDS too (fewer live registers).
template <int D>
__device__ __forceinline__ f32x4 dot_tile16_ll(const uint16_t* arow, const uint16_t* brow, int g) {
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag<D>(arow, kk, g), lds_frag<D>(brow, kk, g), acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ bf16x8 pack8(const float (&x)[2][4]) {
  u32x4 p;
  p[0] = pack_bf16x2(x[0][0], x[0][1]);
  p[1] = pack_bf16x2(x[0][2], x[0][3]);
  p[2] = pack_bf16x2(x[1][0], x[1][1]);
  p[3] = pack_bf16x2(x[1][2], x[1][3]);
  return __builtin_bit_cast(bf16x8, p);
}

// Transposed operand (16 features x 32 rows) from row-major LDS rows: lane
// (g, c16) gets feature 16dt + c16 of rows r0 + 4g + 0..3 and r0 + 16 + 4g + 0..3.
template <int D>
__device__ __forceinline__ bf16x8 lds_frag_t(const uint16_t* base, int r0, int dt, int g, int c16) {
  constexpr int kP = BwdTile16<D>::kPitch;
  const uint16_t* p = base + (r0 + 4 * g + (c16 >> 2)) * kP + 4 * (c16 & 3) + 16 * dt;
  const u32x2 lo = lds_read_tr16(p);
  const u32x2 hi = lds_read_tr16(p + 16 * kP);
  u32x4 a;
  a[0] = lo[0];
  a[1] = lo[1];
  a[2] = hi[0];
  a[3] = hi[1];
  return __builtin_bit_cast(bf16x8, a);
}

// z pass (bf16): grid (runs, bh * n_rounds).  A workgroup walks `run`
// consecutive chunks of one (batch*head, round) segment, keeping the previous
// chunk's rows in LDS and taking the queries' fragments from the same LDS
// rows, so every row is gathered once per round (a workgroup per chunk would
// gather it three times: as a key of its own chunk, of the next chunk, and as
// a query); the next chunk's rows are loaded into registers while the current
// one is computed.  Wavefront w owns queries 16w..16w+15 of the chunk; z2 =
// log2 sum_j 2^(s_ij * scale_log2) over the valid window keys (-inf when
// there is none).
template <int D>
struct alignas(16) ZRunLds {
  static constexpr int kP = D + 16;   // bf16 per row, as BwdTile16
  uint16_t qk[2][kBT * kP];           // chunk c in slot c & 1
  int pos[2][kBT];
};

template <int D>
__global__ __launch_bounds__(256) void bwd_zrun16_kernel(const uint16_t* __restrict__ qk,
                                                         const int32_t* __restrict__ perm_all, BwdShape s, int run,
                                                         float* __restrict__ z2_rounds) {
  __shared__ ZRunLds<D> sh;
  constexpr int kP = ZRunLds<D>::kP;
  constexpr int kPieces = kBT * (D / 8);
  constexpr int kPer = kPieces / 256;   // 16-byte pieces per thread and chunk
  const int seg = blockIdx.y;
  const int L = s.seq_len;
  const int32_t* perm = perm_all + static_cast<size_t>(seg) * L;
  const size_t row0 = static_cast<size_t>(seg / s.n_rounds) * L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int qrow = 16 * wave + c16;
  const int c0 = blockIdx.x * run;
  const int c1 = min(c0 + run, s.n_chunks) - 1;

  u32x4 pr[kPer];
  int ppos = 0;
  auto load = [&](int c) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = threadIdx.x + 256 * i;
      pr[i] = *reinterpret_cast<const u32x4*>(qk + (row0 + perm[c * kBT + u / (D / 8)]) * D + 8 * (u % (D / 8)));
    }
    if (threadIdx.x < kBT) ppos = perm[c * kBT + threadIdx.x];
  };
  auto store = [&](int c) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = threadIdx.x + 256 * i;
      *reinterpret_cast<u32x4*>(&sh.qk[c & 1][(u / (D / 8)) * kP + 8 * (u % (D / 8))]) = pr[i];
    }
    if (threadIdx.x < kBT) sh.pos[c & 1][threadIdx.x] = ppos;
  };
  if (c0 > 0) {
    load(c0 - 1);
    store(c0 - 1);
  }
  load(c0);
  store(c0);
  __syncthreads();

  for (int c = c0; c <= c1; ++c) {
    const bool more = c < c1;
    if (more) load(c + 1);
    const int qslot = c * kBT + qrow;
    const int qpos = sh.pos[c & 1][qrow];
    bf16x8 qf[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qf[kk] = lds_frag<D>(&sh.qk[c & 1][qrow * kP], kk, g);
    float mrun = -INFINITY, lrun = 0.0f;
    for (int h = (c > 0 ? 0 : 1); h < 2; ++h) {
      const int kc = c - 1 + h;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x4 acc = dot_tile16<D>(&sh.qk[kc & 1][(16 * kt + c16) * kP], qf, g);   // S^T[key 16kt+4g+j][query c16]
        float tmax = -INFINITY;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 16 * kt + 4 * g + j;
          bool ok = kc * kBT + kr != qslot;
          if (s.causal) ok = ok && sh.pos[kc & 1][kr] < qpos;
          v[j] = ok ? acc[j] * s.scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, v[j]);
        }
        const float mnew = fmaxf(mrun, tmax);
        if (mnew != -INFINITY) {
          float add = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) add += exp2f(v[j] - mnew);
          lrun = lrun * exp2f(mrun - mnew) + add;
          mrun = mnew;
        }
      }
    }
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const float om = shfl_xor_f(mrun, off), ol = shfl_xor_f(lrun, off);
      const float mnew = fmaxf(mrun, om);
      if (mnew != -INFINITY) {
        lrun = lrun * exp2f(mrun - mnew) + ol * exp2f(om - mnew);
        mrun = mnew;
      }
    }
    if (g == 0) z2_rounds[static_cast<size_t>(seg) * L + qpos] = (mrun == -INFINITY) ? -INFINITY : mrun + log2f(lrun);
    __syncthreads();
    if (more) store(c + 1);   // into chunk c - 1's slot
    __syncthreads();
  }
}

// ------------------------------------------------ fused bf16 backward ----
// One workgroup of 8 wavefronts per run of `run` consecutive chunks of one
// (batch*head), for one round (run chosen by fused_run_length).  Step q brings chunk q's rows (qk, v, dout,
// gathered through perm; the perm entries themselves one step earlier) into
// LDS once, next to chunk q-1's qk and v, and does both halves of the work on
// them.  Wavefronts 0-3 take the query role and 4-7 the key role for row slab
// w % 4 (16 rows of a chunk):
//   query role: queries of chunk q; dq over the keys of chunks q-1 and q (as
//     the query pass above), added to the rows at the end of the step;
//   key role: keys of chunk q-1, then of chunk q.  The queries of chunk q
//     finish chunk q-1's dk and dv (its other queries, chunk q-1, came one
//     step earlier), the rows are written, and the same registers start chunk
//     q's (as the key pass above).
// A run also reads the chunk before it (keys of its first
// query chunk, no key-role output) and takes the chunk after it (key role
// only, to finish its last chunk), so every gradient row of a round has one
// writing workgroup.  A row's dq (step q) is finished one step before its dk
// (step q + 1): the query role leaves dq in LDS and the key role adds it to
// dk, so each row's dqk is read and written once per round (only written in
// round 0).  Compared with the separate passes every row is read once per
// round instead of three times.
//
// Run length: a run loads two chunks beyond its own (the one before, the one
// after), and one workgroup fills a CU, so a launch takes about
// ceil(workgroups / CUs) x (run + 2) chunk-steps; the host picks the run
// length in {8, 16, 32} that minimises it (measured: 32 at 64K text and 512K
// tokens, 16 at the 12K image shape, 3-7 % faster than a fixed 8).
int fused_run_length(int n_chunks, int bh, int n_cu) {
  int best = 8;
  long long best_cost = -1;
  for (int run : {8, 16, 32}) {
    const long long wgs = static_cast<long long>((n_chunks + run - 1) / run) * bh;
    const long long cost = ((wgs + n_cu - 1) / n_cu) * (run + 2);
    if (best_cost < 0 || cost < best_cost) {
      best = run;
      best_cost = cost;
    }
  }
  return best;
}

template <int D>
struct alignas(16) FusedLds {
  static constexpr int kP = D + 16;   // bf16 per row, as BwdTile16
  uint16_t qk[2][kBT * kP];           // chunk c in slot c & 1
  uint16_t v[2][kBT * kP];
  uint16_t dout[kBT * kP];            // the current query chunk
  int pos[2][kBT];
  float z2[kBT];                      // Z (log2 domain) and D of the current query chunk
  float dd[kBT];
  // dq of query chunk c (scaled), slot c & 1, as the query-role lanes hold it:
  // [wavefront][16-feature tile][lane]; the key-role lane of the same row
  // (wavefront + 4, same lane) reads the same entries.
  f32x4 dq[2][4][D / 16][64];
};

// One chunk's rows in flight in registers (loaded during a step, stored to LDS
// after its closing barrier): one 16-byte piece of each matrix per thread.
template <int D, int T>
struct FusedPrefetch {
  static constexpr int kThreads = T;
  static constexpr int kPieces = kBT * (D / 8);
  static constexpr int kPer = (kPieces + T - 1) / T;   // pieces per thread and matrix
  u32x4 q[kPer], v[kPer], o[kPer];
  int pos;
  float z2, dd;
  int prow[kPer];   // perm entries of this thread's rows for the chunk to be loaded next
  int ppos;         // (threads < 64) perm entry of row threadIdx.x of that chunk
};

// perm entries that fused_load needs for chunk c, loaded one step ahead so the
// row gathers do not wait on them.
template <int D, class PF>
__device__ __forceinline__ void fused_perm(PF& f, const int32_t* __restrict__ perm, int c) {
#pragma unroll
  for (int i = 0; i < PF::kPer; ++i) {
    const int u = threadIdx.x + PF::kThreads * i;
    if (u < PF::kPieces) f.prow[i] = perm[c * kBT + u / (D / 8)];
  }
  if (threadIdx.x < kBT) f.ppos = perm[c * kBT + threadIdx.x];
}

// Rows of the chunk whose perm entries fused_perm put in f.
template <int D, class PF>
__device__ __forceinline__ void fused_load(PF& f, const uint16_t* __restrict__ qk,
                                           const uint16_t* __restrict__ vv, const uint16_t* __restrict__ dout,
                                           const float* __restrict__ z2, const float* __restrict__ dd, size_t row0,
                                           bool with_dout) {
#pragma unroll
  for (int i = 0; i < PF::kPer; ++i) {
    const int u = threadIdx.x + PF::kThreads * i;
    if (u < PF::kPieces) {
      const size_t off = (row0 + f.prow[i]) * D + 8 * (u % (D / 8));
      f.q[i] = *reinterpret_cast<const u32x4*>(qk + off);
      f.v[i] = *reinterpret_cast<const u32x4*>(vv + off);
      if (with_dout) f.o[i] = *reinterpret_cast<const u32x4*>(dout + off);
    }
  }
  if (threadIdx.x < kBT) {
    f.pos = f.ppos;
    if (with_dout) {
      f.z2 = z2[row0 + f.pos];
      f.dd = dd[row0 + f.pos];
    }
  }
}

template <int D, class PF>
__device__ __forceinline__ void fused_store(const PF& f, FusedLds<D>& sh, int c, bool with_dout) {
  constexpr int kP = FusedLds<D>::kP;
  const int slot = c & 1;
#pragma unroll
  for (int i = 0; i < PF::kPer; ++i) {
    const int u = threadIdx.x + PF::kThreads * i;
    if (u < PF::kPieces) {
      const int row = u / (D / 8), pc = u % (D / 8);
      *reinterpret_cast<u32x4*>(&sh.qk[slot][row * kP + 8 * pc]) = f.q[i];
      *reinterpret_cast<u32x4*>(&sh.v[slot][row * kP + 8 * pc]) = f.v[i];
      if (with_dout) *reinterpret_cast<u32x4*>(&sh.dout[row * kP + 8 * pc]) = f.o[i];
    }
  }
  if (threadIdx.x < kBT) {
    sh.pos[slot][threadIdx.x] = f.pos;
    if (with_dout) {
      sh.z2[threadIdx.x] = f.z2;
      sh.dd[threadIdx.x] = f.dd;
    }
  }
}

constexpr int kFusedThreads = 512;

template <int D>
__global__ __launch_bounds__(kFusedThreads) void bwd_fused16_kernel(
    const uint16_t* __restrict__ qk, const uint16_t* __restrict__ vv, const uint16_t* __restrict__ dout,
    const int32_t* __restrict__ perm_all, BwdShape s, int round, const float* __restrict__ z2,
    const float* __restrict__ dd, float* __restrict__ dqk, float* __restrict__ dv, int run) {
  __shared__ FusedLds<D> sh;
  constexpr int kP = FusedLds<D>::kP;
  constexpr int kFull = D / 16;            // 16-feature gradient tiles of a row
  using PF = FusedPrefetch<D, kFusedThreads>;
  const int bh = blockIdx.y;
  const int L = s.seq_len;
  const int32_t* perm = perm_all + (static_cast<size_t>(bh) * s.n_rounds + round) * L;
  const size_t row0 = static_cast<size_t>(bh) * L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const bool key_role = wave >= 4;
  const int own = 16 * (wave & 3) + c16;   // this lane's row (query or key) inside a chunk
  const int c0 = blockIdx.x * run;
  const int c1 = min(c0 + run, s.n_chunks) - 1;
  const int q_end = min(c1 + 1, s.n_chunks - 1);

  PF pf;
  if (c0 > 0) {
    fused_perm<D, PF>(pf, perm, c0 - 1);
    fused_load<D, PF>(pf, qk, vv, dout, z2, dd, row0, false);
    fused_store<D, PF>(pf, sh, c0 - 1, false);
  }
  fused_perm<D, PF>(pf, perm, c0);
  fused_load<D, PF>(pf, qk, vv, dout, z2, dd, row0, true);
  fused_store<D, PF>(pf, sh, c0, true);
  if (c0 < q_end) fused_perm<D, PF>(pf, perm, c0 + 1);
  __syncthreads();

  // acc_a: dq (query role) or dv (key role); acc_b: dk (key role); old_*: the
  // rows' current values.
  f32x4 acc_a[kFull], acc_b[kFull], old_a[kFull], old_b[kFull];
#pragma unroll
  for (int i = 0; i < kFull; ++i) {
    acc_a[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    acc_b[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Key role, one (key chunk kc, query chunk q) block: S and dP for 64 queries x
  // this lane's key, then dv^T += dout^T P and dk^T += q^T dS.
  auto key_block = [&](int kc, int q) {
    const uint16_t* krow = &sh.qk[kc & 1][own * kP];
    const uint16_t* vrow = &sh.v[kc & 1][own * kP];
    const int kslot = kc * kBT + own;
    const int kpos = sh.pos[kc & 1][own];
    const uint16_t* qbase = sh.qk[q & 1];
#pragma unroll
    for (int qp = 0; qp < 2; ++qp) {
      float pv[2][4], dsv[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qt = 2 * qp + u;
        const f32x4 sacc = dot_tile16_ll<D>(&qbase[(16 * qt + c16) * kP], krow, g);     // S[query 16qt+4g+j][key c16]
        const f32x4 pacc = dot_tile16_ll<D>(&sh.dout[(16 * qt + c16) * kP], vrow, g);   // dout_q . v_key
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qr = 16 * qt + 4 * g + j;
          bool ok = q * kBT + qr != kslot;
          if (s.causal) ok = ok && kpos < sh.pos[q & 1][qr];
          const float zq = sh.z2[qr];
          const float p = (ok && zq != -INFINITY) ? exp2f(fmaf(sacc[j], s.scale_log2, -zq)) : 0.0f;
          pv[u][j] = p;
          dsv[u][j] = p * (pacc[j] - sh.dd[qr]);
        }
      }
      const bf16x8 bp = pack8(pv), bs = pack8(dsv);
#pragma unroll
      for (int i = 0; i < kFull; ++i) {
        acc_a[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag_t<D>(sh.dout, 32 * qp, i, g, c16), bp,
                                                           acc_a[i], 0, 0, 0);
        acc_b[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag_t<D>(qbase, 32 * qp, i, g, c16), bs,
                                                           acc_b[i], 0, 0, 0);
      }
    }
  };
  // Key role: load the current dv and dqk of chunk kc's rows (nothing in
  // round 0: both start from zero).
  auto key_prefetch = [&](int kc) {
    const int kpos = sh.pos[kc & 1][own];
    const float* dvr = dv + (row0 + kpos) * D;
    const float* dkr = dqk + (row0 + kpos) * D;
#pragma unroll
    for (int i = 0; i < kFull; ++i) {
      const int f = 16 * (i) + 4 * g;
      old_a[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      old_b[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (round != 0) {
        old_a[i] = *reinterpret_cast<const f32x4*>(dvr + f);
        old_b[i] = *reinterpret_cast<const f32x4*>(dkr + f);
      }
    }
  };
  // Key role: chunk kc's dk and dv are complete; add them and chunk kc's dq
  // (left in LDS by the query role) to the rows (plus dout to dv on
  // self-fallback rows in round 0) and clear.
  // (Loading the current values before the block's MFMAs would hide the
  // wait, but the registers it needs make the kernel spill; key_touch below
  // hides part of it with two registers.)
  auto key_store = [&](int kc) {
    const int kpos = sh.pos[kc & 1][own];
    float* dvr = dv + (row0 + kpos) * D;
    float* dkr = dqk + (row0 + kpos) * D;
    const bool fallback = round == 0 && z2[row0 + kpos] == -INFINITY;
#pragma unroll
    for (int i = 0; i < kFull; ++i) {
      const int f = 16 * (i) + 4 * g;
      f32x4 a = old_a[i], b = old_b[i];
      const f32x4 dqv = sh.dq[kc & 1][wave & 3][i][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] += acc_a[i][j];
        b[j] = fmaf(acc_b[i][j], s.scale, b[j] + dqv[j]);
      }
      if (fallback) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] += bf16_to_f32(dout[(row0 + kpos) * D + f + j]);
      }
      *reinterpret_cast<f32x4*>(dvr + f) = a;
      *reinterpret_cast<f32x4*>(dkr + f) = b;
      acc_a[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      acc_b[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  // Key role: one float of each 128-byte line of chunk kc's dv and dqk rows
  // (lanes g = 0..3 of a row take a quarter row each), read before the block's
  // MFMAs so the lines are on their way into the cache when key_prefetch asks
  // for the rows; the values are only consumed by an empty asm statement after
  // key_prefetch.  Touching a step earlier measured slower: the lines leave
  // the cache again before they are read.
  auto key_touch = [&](int kc, float& a, float& b) {
    const int kpos = sh.pos[kc & 1][own];
    const size_t off = (row0 + kpos) * D + (D / 4) * g;
    a = dv[off];
    b = dqk[off];
    asm volatile("" ::: "memory");   // keep the loads ahead of the block
  };
  // Query role, chunk q: dq^T += k^T dS^T over the keys of chunks q-1 and q,
  // left in LDS for the key role, which adds it to the rows with dk.
  auto query_chunk = [&](int q) {
    const uint16_t* qrow = &sh.qk[q & 1][own * kP];
    const uint16_t* orow = &sh.dout[own * kP];
    const int qslot = q * kBT + own;
    const int qpos = sh.pos[q & 1][own];
    const float zq = sh.z2[own];
    const float dq = sh.dd[own];
    for (int kc = (q > 0 ? q - 1 : q); kc <= q; ++kc) {
      const uint16_t* kbase = sh.qk[kc & 1];
      const uint16_t* vbase = sh.v[kc & 1];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        float dsv[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kt = 2 * kp + u;
          const f32x4 sacc = dot_tile16_ll<D>(&kbase[(16 * kt + c16) * kP], qrow, g);   // S^T[key 16kt+4g+j][query c16]
          const f32x4 pacc = dot_tile16_ll<D>(&vbase[(16 * kt + c16) * kP], orow, g);   // v_key . dout_q
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kr = 16 * kt + 4 * g + j;
            bool ok = kc * kBT + kr != qslot;
            if (s.causal) ok = ok && sh.pos[kc & 1][kr] < qpos;
            const float p = (ok && zq != -INFINITY) ? exp2f(fmaf(sacc[j], s.scale_log2, -zq)) : 0.0f;
            dsv[u][j] = p * (pacc[j] - dq);
          }
        }
        const bf16x8 bs = pack8(dsv);
#pragma unroll
        for (int i = 0; i < kFull; ++i)
          acc_a[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag_t<D>(kbase, 32 * kp, i, g, c16), bs, acc_a[i],
                                                             0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < kFull; ++i) {
      f32x4 a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = acc_a[i][j] * s.scale;
      sh.dq[q & 1][wave][i][lane] = a;
      acc_a[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };

  for (int q = c0; q <= q_end; ++q) {
    const bool more = q < q_end;
    if (more) {
      fused_load<D, PF>(pf, qk, vv, dout, z2, dd, row0, true);   // chunk q + 1
      if (q + 2 <= q_end) fused_perm<D, PF>(pf, perm, q + 2);
    }
    if (!key_role) {
      if (q <= c1) query_chunk(q);
    } else {
      if (q - 1 >= c0) {
        float ta = 0.0f, tb = 0.0f;
        if (round != 0) key_touch(q - 1, ta, tb);
        key_block(q - 1, q);
        key_prefetch(q - 1);
        asm volatile("" ::"v"(ta), "v"(tb));   // the touch loads end here, behind the block's MFMAs
        key_store(q - 1);
      }
      if (q <= c1) key_block(q, q);
    }
    __syncthreads();
    if (more) fused_store<D, PF>(pf, sh, q + 1, true);
    __syncthreads();
  }
  // The sequence's last chunk has no following query chunk.
  if (key_role && c1 == s.n_chunks - 1) {
    key_prefetch(c1);
    key_store(c1);
  }
}

template <int D, bool BF16>
hipError_t launch_bwd_typed(const void* qk, const void* v, const void* out, const void* dout, const float* lse,
                            const int32_t* perm, int bh, const BwdShape& s, float* z2_rounds, float* z2, float* dd,
                            float* dqk, float* dv, hipStream_t stream) {
  const uint16_t* q16 = static_cast<const uint16_t*>(qk);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  const uint16_t* o16 = static_cast<const uint16_t*>(dout);
  if (lse == nullptr) {   // per-round normalisers, recomputed
    if constexpr (BF16) {
      // runs of 4 to 16 chunks measured alike; 32 and 64 slower
      const int zrun = std::min(8, s.n_chunks);
      hipLaunchKernelGGL(bwd_zrun16_kernel<D>, dim3((s.n_chunks + zrun - 1) / zrun, bh * s.n_rounds), dim3(256), 0,
                         stream, q16, perm, s, zrun, z2_rounds);
    }
    else
      hipLaunchKernelGGL((bwd_z_kernel<D, false>), dim3(s.n_chunks, bh * s.n_rounds), dim3(256), 0, stream, qk, perm,
                         s, z2_rounds);
  }
  const int n_rows = bh * s.seq_len;
  const int stats_threads = n_rows * (D / 8);
  hipLaunchKernelGGL((bwd_stats_kernel<D, BF16>), dim3((stats_threads + 255) / 256), dim3(256), 0, stream, z2_rounds,
                     lse, out, dout, n_rows, s.seq_len, s.n_rounds, z2, dd);
  int run = 8;
  if constexpr (BF16) {
    int dev = 0, n_cu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
      n_cu = 256;
    run = fused_run_length(s.n_chunks, bh, n_cu);
  }
  for (int r = 0; r < s.n_rounds; ++r) {
    if constexpr (BF16) {
      hipLaunchKernelGGL(bwd_fused16_kernel<D>, dim3((s.n_chunks + run - 1) / run, bh),
                         dim3(kFusedThreads), 0, stream, q16, v16, o16, perm, s, r, z2, dd, dqk, dv, run);
    } else {
      hipLaunchKernelGGL((bwd_key_kernel<D, false>), dim3(s.n_chunks, bh), dim3(256), 0, stream, qk, v, dout, perm, s,
                         r, z2, dd, dqk, dv);
      hipLaunchKernelGGL((bwd_query_kernel<D, false>), dim3(s.n_chunks, bh), dim3(256), 0, stream, qk, v, dout, perm,
                         s, r, z2, dd, dqk);
    }
  }
  return hipGetLastError();
}

}  // namespace

size_t backward_scratch_bytes(int bh, int seq_len, int n_rounds) {
  const size_t n = static_cast<size_t>(bh) * seq_len;
  return align_up(n * n_rounds * sizeof(float), 256) + 2 * align_up(n * sizeof(float), 256);
}

hipError_t launch_attend_backward(const void* qk, const void* v, bool bf16, const int32_t* perm, int bh, int seq_len,
                                  int d, int n_rounds, bool causal, const void* out, const void* dout,
                                  const float* lse, float* dqk, float* dv, void* workspace, hipStream_t stream) {
  BwdShape s{};
  s.seq_len = seq_len;
  s.n_rounds = n_rounds;
  s.n_chunks = seq_len / kBT;
  s.causal = causal ? 1 : 0;
  s.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
  s.scale_log2 = s.scale * kLog2e;
  const size_t n = static_cast<size_t>(bh) * seq_len;
  char* ws = static_cast<char*>(workspace);
  float* z2_rounds = reinterpret_cast<float*>(ws);
  float* z2 = reinterpret_cast<float*>(ws + align_up(n * n_rounds * sizeof(float), 256));
  float* dd = reinterpret_cast<float*>(ws + align_up(n * n_rounds * sizeof(float), 256) + align_up(n * sizeof(float), 256));
  if (d == 64)
    return bf16 ? launch_bwd_typed<64, true>(qk, v, out, dout, lse, perm, bh, s, z2_rounds, z2, dd, dqk, dv, stream)
                : launch_bwd_typed<64, false>(qk, v, out, dout, lse, perm, bh, s, z2_rounds, z2, dd, dqk, dv, stream);
  return bf16 ? launch_bwd_typed<128, true>(qk, v, out, dout, lse, perm, bh, s, z2_rounds, z2, dd, dqk, dv, stream)
              : launch_bwd_typed<128, false>(qk, v, out, dout, lse, perm, bh, s, z2_rounds, z2, dd, dqk, dv, stream);
}

}  // namespace rlsh
