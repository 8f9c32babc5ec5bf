// Position-wise feed-forward layer applied in chunks of positions.
//
// "Reformer: The Efficient Transformer" (research summary), Summary and Key
// points (reversible layers bullet): the feed-forward layers run over a chunk
// of positions at a time, so the d_ff-wide activation is never held for the
// whole sequence, and the results stay the same.  Here y = relu(x W1^T + b1) W2^T + b2 (the
// pages name no activation; ReLU is the plainest reading), with the d_ff-wide
// intermediate of one chunk at a time held in the caller's workspace.
//
// Design for gfx950: one bf16 MFMA GEMM kernel, Y = act(X W^T + b) with X
// [M, K] and W [N, K] both row-major (the layout of a linear layer's weight),
// computed as Y^T tiles D[n][m] = sum_k W[n][k] X[m][k] so that both MFMA
// operands are 16-byte row fragments and each lane ends up with 4 consecutive
// outputs of one row (one 8-byte store).  A workgroup owns 128 x 128 outputs
// (4 wavefronts of 64 x 64 = 4 x 4 tiles of v_mfma_f32_16x16x32_bf16), K is
// streamed in blocks of 64 through double-buffered LDS with a register
// prefetch of the next block.  Every output element is summed over K in the
// same order whatever the number of rows, so chunking changes no bit.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace rlsh {

namespace {

constexpr int kFT = 128;       // rows and columns of a workgroup tile
constexpr int kFK = 64;        // K per LDS block
constexpr int kFPitch = kFK;       // bf16 per LDS row: 8 pieces of 16 bytes, no pad
// Piece p of row r sits in slot p ^ ((r >> 1) & 7): the 16 lanes of an MFMA
// operand read (rows r0 .. r0 + 15, one piece) and of a tile copy store (two
// rows, all eight pieces) each touch 16 different 4-bank groups.
__device__ __forceinline__ int ff_slot(int row, int piece) { return piece ^ ((row >> 1) & 7); }

struct alignas(16) FfLds {
  uint16_t w[2][kFT * kFPitch];
  uint16_t x[2][kFT * kFPitch];
};

// Workgroup -> output tile.  Workgroups are dispatched to the 8 XCDs in turn
// (workgroup b to XCD b % 8), and each XCD has its own L2.  The tile grid is
// cut into pm x pn blocks, one per XCD; an XCD walks its block in groups of
// kFGroup tile rows, sweeping the columns with the rows of a group innermost,
// so the 64 workgroups an XCD holds at once cover about 8 x 8 tiles and a
// group's rows of X stay in L2 for the whole sweep.  pm == 0: row-major order.
constexpr int kFGroup = 8;

struct FfTileOrder {
  int mt, nt;   // tiles along M and N
  int pm, pn;   // XCD blocks along M and N (pm * pn == 8), or pm == 0

  __device__ __forceinline__ void tile_of(int b, int& m, int& n) const {
    if (pm == 0) {
      m = b / nt;
      n = b - m * nt;
      return;
    }
    const int xcd = b & 7, local = b >> 3;
    const int bm = mt / pm, bn = nt / pn;
    const int group = local / (kFGroup * bn), idx = local - group * kFGroup * bn;
    const int gsize = min(kFGroup, bm - group * kFGroup);
    const int ln = idx / gsize, lm = group * kFGroup + (idx - ln * gsize);
    m = (xcd / pn) * bm + lm;
    n = (xcd % pn) * bn + ln;
  }
};

// The even split with the least L2 fill traffic per XCD, counted in tile rows
// of 128 x K: its rows of X once, and its columns of W once if they fit in
// the 4 MB L2, else once per group of rows.
FfTileOrder ff_tile_order(int mt, int nt, int K) {
  FfTileOrder o{mt, nt, 0, 1};
  long best = 0;
  const long tile_bytes = static_cast<long>(kFT) * K * 2;
  for (int pm = 1; pm <= 8; pm *= 2) {
    const int pn = 8 / pm;
    if (mt % pm != 0 || nt % pn != 0) continue;
    const int bm = mt / pm, bn = nt / pn;
    const bool w_fits = bn * tile_bytes <= (4l << 20);
    const long cost = bm + static_cast<long>(bn) * (w_fits ? 1 : (bm + kFGroup - 1) / kFGroup);
    if (best == 0 || cost < best) {
      best = cost;
      o.pm = pm;
      o.pn = pn;
    }
  }
  return o;
}

template <bool RELU>
__global__ __launch_bounds__(256, 2) void linear_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                        const float* __restrict__ bias, int M, int N, int K,
                                                        uint16_t* __restrict__ Y, FfTileOrder order) {
  __shared__ FfLds sh;
  int m_tile, n_tile;
  order.tile_of(blockIdx.x, m_tile, n_tile);
  const int n_blk = n_tile * kFT, m_blk = m_tile * kFT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int wn = 64 * (wave & 1), wm = 64 * (wave >> 1);
  // Tile copy: 128 rows x 64 k = 1024 pieces of 16 bytes per matrix, 4 per thread.
  auto load_block = [&](int k0, u32x4 (&wr)[4], u32x4 (&xr)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = threadIdx.x + 256 * i;
      const int row = u >> 3, pc = u & 7;
      const int xm = min(m_blk + row, M - 1);   // rows past M are computed but never stored
      wr[i] = *reinterpret_cast<const u32x4*>(W + static_cast<size_t>(n_blk + row) * K + k0 + 8 * pc);
      xr[i] = *reinterpret_cast<const u32x4*>(X + static_cast<size_t>(xm) * K + k0 + 8 * pc);
    }
  };
  auto store_block = [&](int buf, const u32x4 (&wr)[4], const u32x4 (&xr)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = threadIdx.x + 256 * i;
      const int row = u >> 3, pc = u & 7;
      *reinterpret_cast<u32x4*>(&sh.w[buf][row * kFPitch + 8 * ff_slot(row, pc)]) = wr[i];
      *reinterpret_cast<u32x4*>(&sh.x[buf][row * kFPitch + 8 * ff_slot(row, pc)]) = xr[i];
    }
  };

  f32x4 acc[4][4];   // [n subtile][m subtile]: lane holds D[n 16i + 4g + j][m 16t + c16]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4 wr[4], xr[4];
  load_block(0, wr, xr);
  store_block(0, wr, xr);
  __syncthreads();
  const int n_kb = K / kFK;
  for (int kb = 0; kb < n_kb; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < n_kb;
    if (more) load_block((kb + 1) * kFK, wr, xr);
#pragma unroll
    for (int ks = 0; ks < kFK / 32; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               &sh.w[buf][(wn + 16 * i + c16) * kFPitch + 8 * ff_slot(c16, 4 * ks + g)]));
        bfr[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                &sh.x[buf][(wm + 16 * i + c16) * kFPitch + 8 * ff_slot(c16, 4 * ks + g)]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[t], acc[i][t], 0, 0, 0);
    }
    if (more) store_block(buf ^ 1, wr, xr);
    __syncthreads();
  }

  // Epilogue: bias, activation, bf16, 4 consecutive outputs of one row per store.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n_blk + wn + 16 * i + 4 * g;
    const f32x4 b = *reinterpret_cast<const f32x4*>(bias + n);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = m_blk + wm + 16 * t + c16;
      if (m >= M) continue;
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[j] = acc[i][t][j] + b[j];
        if (RELU) y[j] = fmaxf(y[j], 0.0f);
      }
      u32x2 pk;
      pk[0] = pack_bf16x2(y[0], y[1]);
      pk[1] = pack_bf16x2(y[2], y[3]);
      *reinterpret_cast<u32x2*>(Y + static_cast<size_t>(m) * N + n) = pk;
    }
  }
}

template <bool RELU>
void launch_linear(const uint16_t* X, const uint16_t* W, const float* bias, int M, int N, int K, uint16_t* Y,
                   hipStream_t stream) {
  const int mt = (M + kFT - 1) / kFT, nt = N / kFT;
  hipLaunchKernelGGL((linear_kernel<RELU>), dim3(mt * nt), dim3(256), 0, stream, X, W, bias, M, N, K, Y,
                     ff_tile_order(mt, nt, K));
}

}  // namespace

size_t feed_forward_chunk(int n_tokens, int chunk_tokens) {
  return static_cast<size_t>(chunk_tokens <= 0 ? n_tokens : std::min(chunk_tokens, n_tokens));
}

hipError_t launch_feed_forward(const uint16_t* x, const uint16_t* w1, const float* b1, const uint16_t* w2,
                               const float* b2, int n_tokens, int d_model, int d_ff, int chunk_tokens, uint16_t* out,
                               uint16_t* hidden, hipStream_t stream) {
  const int chunk = static_cast<int>(feed_forward_chunk(n_tokens, chunk_tokens));
  for (int t0 = 0; t0 < n_tokens; t0 += chunk) {
    const int rows = std::min(chunk, n_tokens - t0);
    launch_linear<true>(x + static_cast<size_t>(t0) * d_model, w1, b1, rows, d_ff, d_model, hidden, stream);
    launch_linear<false>(hidden, w2, b2, rows, d_model, d_ff, out + static_cast<size_t>(t0) * d_model, stream);
  }
  return hipGetLastError();
}

}  // namespace rlsh
