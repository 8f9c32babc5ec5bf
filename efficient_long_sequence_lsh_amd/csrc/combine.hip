// Stage 5: combine the hash rounds with logsumexp weights and apply the self
// fallback; rows are already in sequence order (the attention stage stores
// by original position).
//
// out_i = sum_r exp(z_r(i) - Z_i) o_r(i),  Z_i = logsumexp_r z_r(i).
// If every z_r(i) is -inf the position had no valid non-self target in any
// round, so it attends to itself and out_i = v_i ("Reformer: The Efficient
// Transformer" (research summary), Key points, Shared-QK bullet).  Combining
// with logsumexp weights is the reading taken for how the rounds ("Number of
// hash rounds" bullet) are merged: it equals one softmax over the keys of all
// rounds together.
//
// Pure HBM stream: r * (4d + 4) bytes read and d * e written per row.  Each
// thread owns 4 consecutive features (16-byte loads), d/4 threads per row.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>
#include <cmath>

namespace rlsh {

namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o, const float* __restrict__ z,
                                                      const void* __restrict__ v_raw, int n_rows, int seq_len,
                                                      int n_rounds, void* __restrict__ out_raw,
                                                      float* __restrict__ lse) {
  constexpr int kTpr = D / 4;                 // threads per row
  constexpr int kRowsPerBlock = 256 / kTpr;
  const int sub = threadIdx.x % kTpr;
  const int rsub = threadIdx.x / kTpr;
  for (int row = blockIdx.x * kRowsPerBlock + rsub; row < n_rows; row += gridDim.x * kRowsPerBlock) {
    const int bh = row / seq_len;
    const int pos = row - bh * seq_len;
    const size_t zrow = static_cast<size_t>(bh) * n_rounds * seq_len + pos;   // round 0
    float zmax = -INFINITY;
    for (int r = 0; r < n_rounds; ++r) zmax = fmaxf(zmax, z[zrow + static_cast<size_t>(r) * seq_len]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float row_lse = -INFINITY;
    if (zmax == -INFINITY) {
      if constexpr (BF16) {
        const uint16_t* vv = static_cast<const uint16_t*>(v_raw) + static_cast<size_t>(row) * D + 4 * sub;
        const u32x2 raw = *reinterpret_cast<const u32x2*>(vv);
        acc[0] = __uint_as_float(raw[0] << 16);
        acc[1] = __uint_as_float(raw[0] & 0xffff0000u);
        acc[2] = __uint_as_float(raw[1] << 16);
        acc[3] = __uint_as_float(raw[1] & 0xffff0000u);
      } else {
        acc = *reinterpret_cast<const f32x4*>(static_cast<const float*>(v_raw) + static_cast<size_t>(row) * D + 4 * sub);
      }
    } else {
      float wsum = 0.0f;
      for (int r = 0; r < n_rounds; ++r) {
        const size_t zi = zrow + static_cast<size_t>(r) * seq_len;
        const float w = expf(z[zi] - zmax);      // 0 for rounds without a target
        wsum += w;
        if (w > 0.0f) {
          const f32x4 ov = *reinterpret_cast<const f32x4*>(o + zi * D + 4 * sub);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] = fmaf(w, ov[j], acc[j]);
        }
      }
      const float inv = 1.0f / wsum;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] *= inv;
      row_lse = zmax + logf(wsum);
    }
    if (lse != nullptr && sub == 0) lse[row] = row_lse;
    if constexpr (BF16) {
      u32x2 packed;
      packed[0] = pack_bf16x2(acc[0], acc[1]);
      packed[1] = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out_raw) + static_cast<size_t>(row) * D + 4 * sub) = packed;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out_raw) + static_cast<size_t>(row) * D + 4 * sub) = acc;
    }
  }
}

template <int D, bool BF16>
hipError_t launch_typed(const float* o, const float* z, const void* v, int n_rows, int seq_len, int n_rounds,
                        void* out, float* lse, hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / (D / 4);
  int blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  blocks = std::max(1, std::min(blocks, 256 * 32));
  hipLaunchKernelGGL((combine_kernel<D, BF16>), dim3(blocks), dim3(256), 0, stream, o, z, v, n_rows, seq_len, n_rounds,
                     out, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float* o_rounds, const float* z_rounds, const void* v, bool bf16, int bh, int seq_len,
                          int d, int n_rounds, void* out, float* lse, hipStream_t stream) {
  const int n_rows = bh * seq_len;
  if (d == 64)
    return bf16 ? launch_typed<64, true>(o_rounds, z_rounds, v, n_rows, seq_len, n_rounds, out, lse, stream)
                : launch_typed<64, false>(o_rounds, z_rounds, v, n_rows, seq_len, n_rounds, out, lse, stream);
  return bf16 ? launch_typed<128, true>(o_rounds, z_rounds, v, n_rows, seq_len, n_rounds, out, lse, stream)
              : launch_typed<128, false>(o_rounds, z_rounds, v, n_rows, seq_len, n_rounds, out, lse, stream);
}

}  // namespace rlsh
