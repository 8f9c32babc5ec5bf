// Launchers shared between the kernel sources and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rlsh {

// Geometry of the hash stage (all derived on the host from the ABI arguments).
struct HashShape {
  int n_tokens;    // batch * heads * seq_len
  int seq_len;
  int d;           // 64 or 128
  int n_rounds;
  int n_buckets;   // even, >= 2
  int half;        // n_buckets / 2
  int n_ctiles;    // ceil(half / 32): column tiles of 32 rotation columns
  int code_bits;   // bits of the candidate code packed into a projection key
  int group_log2;  // MFMA path: a key group spans 2^group_log2 consecutive column tiles
};

HashShape make_hash_shape(int batch, int heads, int seq_len, int d, int n_rounds, int n_buckets);

// Byte sizes of the hash scratch regions, in workspace order.
struct HashScratch {
  size_t frag_bytes;     // rotation fragments: bf16 R_hi and block-scaled fp6 R_lo per 32-column tile
  size_t rt_bytes;       // rotations transposed to float32 [round][column][k]
  size_t bound_bytes;    // per-tile column-norm maxima of the error-bound terms (float bits)
  size_t counter_bytes;  // near-tie counter
  size_t list_bytes;     // near-tie list (3 int32 per entry, capacity n_tokens * n_rounds)
  size_t total;
};
HashScratch hash_scratch(const HashShape& s);

// marks (optional, may be null): events recorded after the set-up kernels, after the
// projection/argmax kernel and after the near-tie fix-up.
hipError_t launch_hash(const void* qk, bool bf16, const float* rotations, const HashShape& s,
                       int32_t* buckets, int32_t* n_near_ties, void* workspace, hipStream_t stream,
                       hipEvent_t* marks = nullptr);
hipError_t launch_fill_zero_buckets(int32_t* buckets, size_t n, hipStream_t stream);

constexpr int kMaxSortKeyBits = 14;   // bucket ids below 2^14

struct SortShape {
  int n_seg;         // batch * heads * n_rounds
  int seq_len;
  int n_buckets;
  int n_tiles;       // ceil(seq_len / 4096): tile workgroups per segment
  int key_bits;      // ceil(log2(n_buckets))
  int n_bins;        // bins of the tile passes: n_buckets, or coarse bins of two passes
  int bin_bits;      // bits of a bin
  int bin_shift;     // bin = bucket >> bin_shift; two passes: the low bits sorted second
  int pos_bits;      // two passes: bits of a position in a 32-bit entry
  bool block;        // one workgroup per segment (short segments, few buckets)
  bool two_pass;     // coarse tile pass, then one workgroup per (segment, coarse bin)
  bool wide_entries; // two passes with 64-bit entries (low bits and position do not fit 32)
};
SortShape make_sort_shape(int n_seg, int seq_len, int n_buckets);
size_t sort_scratch_bytes(const SortShape& s);
hipError_t launch_sort(const int32_t* buckets, const SortShape& s, int32_t* perm, int32_t* inv,
                       void* workspace, hipStream_t stream);

hipError_t launch_chunk_attend(const void* qk, const void* v, bool bf16, const int32_t* perm,
                               int bh, int seq_len, int d, int n_rounds, int chunk_len, bool causal,
                               float* o_rounds, float* z_rounds, hipStream_t stream);

// lse (optional): per position, the log of the combined softmax normaliser
// over every round's targets (-inf on self-fallback rows).
hipError_t launch_combine(const float* o_rounds, const float* z_rounds, const void* v, bool bf16,
                          int bh, int seq_len, int d, int n_rounds, void* out, float* lse, hipStream_t stream);

// Compact per-round intermediates for the bf16 pipeline with 64-slot chunks:
// o as float16 (d = 64) or 12-bit block floating point (d = 128) rows that
// carry their own z and scale exponent in the lowest bits of their values
// (192 bytes per row at d = 128, 2d bytes at d = 64).  Rounds
// 0..r-2 are stored compact; the last round's launch combines all rounds in
// place and writes `out` (mark, optional: event recorded between the two).
bool compact_rounds_supported(bool bf16, int seq_len, int chunk_len);
hipError_t launch_attend_combine_compact(const void* qk, const void* v, const int32_t* perm, int bh, int seq_len,
                                         int d, int n_rounds, bool causal, uint16_t* o16, void* out,
                                         float* lse, hipStream_t stream, hipEvent_t* mark);

// Local (sliding-chunk) attention over separate q, k, v; out in the input dtype.
hipError_t launch_local_attend(const void* q, const void* k, const void* v, bool bf16, int bh, int seq_len, int d,
                               int chunk_len, int n_before, int n_after, bool causal, void* out, hipStream_t stream);

// Gradients of chunk attention + combine for a given sorted order (chunks of
// 64 slots): dqk, dv float32 [bh, L, d]; workspace backward_scratch_bytes().
size_t backward_scratch_bytes(int bh, int seq_len, int n_rounds);
// lse (optional): the forward's per-position log normaliser; when given the
// normaliser pass is skipped.
hipError_t launch_attend_backward(const void* qk, const void* v, bool bf16, const int32_t* perm, int bh, int seq_len,
                                  int d, int n_rounds, bool causal, const void* out, const void* dout,
                                  const float* lse, float* dqk, float* dv, void* workspace, hipStream_t stream);

// Position-wise feed-forward y = relu(x W1^T + b1) W2^T + b2 in chunks of
// positions (bf16 x, weights and y; float32 biases); hidden holds one chunk's
// [chunk, d_ff] bf16 intermediate.
size_t feed_forward_chunk(int n_tokens, int chunk_tokens);
hipError_t launch_feed_forward(const uint16_t* x, const uint16_t* w1, const float* b1, const uint16_t* w2,
                               const float* b2, int n_tokens, int d_model, int d_ff, int chunk_tokens, uint16_t* out,
                               uint16_t* hidden, hipStream_t stream);

}  // namespace rlsh
