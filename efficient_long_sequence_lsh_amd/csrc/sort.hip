// Stage 2: stable sort of each (batch, head, round) segment by bucket id.
//
// "Reformer: The Efficient Transformer" (research summary), Summary: positions
// are sorted by bucket so that similar vectors become neighbours; Key points,
// LSH attention bullet: chunks are cut from the sorted order.  Ties keep the
// original position order (stable), so the permutation is unique.
//
// Design for gfx950: bucket ids are small integers (< 2^14), so one counting
// pass replaces a comparison sort.  A segment is cut into tiles; one
// wavefront owns a tile and walks it in position order, 64 keys at a time.
// Equal keys inside a group of 64 are found with one ballot per key bit (the
// lanes that agree on every bit share a key), so each distinct key costs one
// LDS update by its lowest lane and ranks inside the group come from a
// popcount -- no LDS atomics, no contention on skewed buckets.
//   hist:    per-tile bucket counts, layout [segment][tile][bucket]
//   scan1:   exclusive prefix over tiles per bucket, totals per bucket
//   scan2:   exclusive prefix over buckets of the totals
//   scatter: slot = bucket base + earlier tiles + rank inside the tile;
//            perm[slot] = position, inv[position] = slot.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace rlsh {

namespace {

__device__ __forceinline__ uint64_t match_key(int key, bool active, int key_bits) {
  uint64_t peers = __ballot(active);
  for (int bit = 0; bit < key_bits; ++bit) {
    bool set = (key >> bit) & 1;
    uint64_t bal = __ballot(active && set);
    peers &= set ? bal : ~bal;
  }
  return peers;
}

__global__ __launch_bounds__(64) void sort_hist_kernel(const int32_t* __restrict__ buckets, SortShape s,
                                                       int32_t* __restrict__ counts) {
  extern __shared__ int32_t cnt[];
  const int t = blockIdx.x, seg = blockIdx.y, lane = threadIdx.x;
  for (int k = lane; k < s.n_buckets; k += 64) cnt[k] = 0;
  __syncthreads();
  const int32_t* keys = buckets + static_cast<size_t>(seg) * s.seq_len;
  const int p0 = t * s.tile, p1 = min(s.seq_len, p0 + s.tile);
  for (int base = p0; base < p1; base += 64) {
    const int pos = base + lane;
    const bool act = pos < p1;
    const int key = act ? keys[pos] : 0;
    const uint64_t peers = match_key(key, act, s.key_bits);
    const uint64_t lower = peers & ((1ull << lane) - 1ull);
    if (act && lower == 0ull) cnt[key] += __popcll(peers);
  }
  __syncthreads();
  int32_t* out = counts + (static_cast<size_t>(seg) * s.n_tiles + t) * s.n_buckets;
  for (int k = lane; k < s.n_buckets; k += 64) out[k] = cnt[k];
}

// Per bucket: exclusive prefix over tiles (in place) and the bucket total.
__global__ __launch_bounds__(256) void sort_scan_tiles_kernel(int32_t* __restrict__ counts, SortShape s,
                                                              int32_t* __restrict__ totals) {
  const int seg = blockIdx.y;
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= s.n_buckets) return;
  int32_t* c = counts + static_cast<size_t>(seg) * s.n_tiles * s.n_buckets + k;
  int run = 0;
  for (int t = 0; t < s.n_tiles; ++t) {
    int v = c[static_cast<size_t>(t) * s.n_buckets];
    c[static_cast<size_t>(t) * s.n_buckets] = run;
    run += v;
  }
  totals[static_cast<size_t>(seg) * s.n_buckets + k] = run;
}

// Exclusive prefix over buckets of the totals (in place), one block per segment.
__global__ __launch_bounds__(1024) void sort_scan_buckets_kernel(int32_t* __restrict__ totals, SortShape s) {
  __shared__ int32_t part[1024];
  const int seg = blockIdx.x, tid = threadIdx.x;
  const int per = (s.n_buckets + 1023) / 1024;
  const int k0 = min(s.n_buckets, tid * per), k1 = min(s.n_buckets, k0 + per);
  int32_t* tv = totals + static_cast<size_t>(seg) * s.n_buckets;
  int sum = 0;
  for (int k = k0; k < k1; ++k) sum += tv[k];
  part[tid] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan over 1024 partial sums.
  for (int off = 1; off < 1024; off <<= 1) {
    int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int k = k0; k < k1; ++k) {
    int v = tv[k];
    tv[k] = run;
    run += v;
  }
}

__global__ __launch_bounds__(64) void sort_scatter_kernel(const int32_t* __restrict__ buckets, SortShape s,
                                                          const int32_t* __restrict__ tile_off,
                                                          const int32_t* __restrict__ bucket_base,
                                                          int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  extern __shared__ int32_t cur[];
  const int t = blockIdx.x, seg = blockIdx.y, lane = threadIdx.x;
  const int32_t* off = tile_off + (static_cast<size_t>(seg) * s.n_tiles + t) * s.n_buckets;
  const int32_t* bb = bucket_base + static_cast<size_t>(seg) * s.n_buckets;
  for (int k = lane; k < s.n_buckets; k += 64) cur[k] = bb[k] + off[k];
  __syncthreads();
  const size_t seg_base = static_cast<size_t>(seg) * s.seq_len;
  const int32_t* keys = buckets + seg_base;
  const int p0 = t * s.tile, p1 = min(s.seq_len, p0 + s.tile);
  for (int base = p0; base < p1; base += 64) {
    const int pos = base + lane;
    const bool act = pos < p1;
    const int key = act ? keys[pos] : 0;
    const uint64_t peers = match_key(key, act, s.key_bits);
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    const int start = act ? cur[key] : 0;
    if (act && rank == 0) cur[key] = start + __popcll(peers);
    if (act) {
      const int slot = start + rank;
      perm[seg_base + slot] = pos;
      if (inv != nullptr) inv[seg_base + pos] = slot;
    }
  }
}

__global__ void iota_kernel(int32_t* __restrict__ perm, int32_t* __restrict__ inv, int n_seg, int seq_len) {
  const size_t n = static_cast<size_t>(n_seg) * seq_len;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    int pos = static_cast<int>(i % seq_len);
    perm[i] = pos;
    if (inv != nullptr) inv[i] = pos;
  }
}

}  // namespace

SortShape make_sort_shape(int n_seg, int seq_len, int n_buckets) {
  SortShape s{};
  s.n_seg = n_seg;
  s.seq_len = seq_len;
  s.n_buckets = n_buckets;
  int tile = 1024;
  while (tile < 2 * n_buckets) tile <<= 1;
  s.tile = tile;
  s.n_tiles = (seq_len + tile - 1) / tile;
  int kb = 0;
  while ((1 << kb) < n_buckets) ++kb;
  s.key_bits = kb;
  return s;
}

size_t sort_scratch_bytes(const SortShape& s) {
  if (s.n_buckets <= 1) return 0;
  size_t off = align_up(static_cast<size_t>(s.n_seg) * s.n_tiles * s.n_buckets * sizeof(int32_t), 256);
  size_t tot = align_up(static_cast<size_t>(s.n_seg) * s.n_buckets * sizeof(int32_t), 256);
  return off + tot;
}

hipError_t launch_sort(const int32_t* buckets, const SortShape& s, int32_t* perm, int32_t* inv, void* workspace,
                       hipStream_t stream) {
  if (s.n_buckets <= 1) {
    size_t n = static_cast<size_t>(s.n_seg) * s.seq_len;
    unsigned grid = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 8192));
    hipLaunchKernelGGL(iota_kernel, dim3(std::max(grid, 1u)), dim3(256), 0, stream, perm, inv, s.n_seg, s.seq_len);
    return hipGetLastError();
  }
  char* ws = static_cast<char*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  int32_t* totals = reinterpret_cast<int32_t*>(
      ws + align_up(static_cast<size_t>(s.n_seg) * s.n_tiles * s.n_buckets * sizeof(int32_t), 256));
  const size_t lds = static_cast<size_t>(s.n_buckets) * sizeof(int32_t);
  dim3 tg(s.n_tiles, s.n_seg);
  hipLaunchKernelGGL(sort_hist_kernel, tg, dim3(64), lds, stream, buckets, s, counts);
  hipLaunchKernelGGL(sort_scan_tiles_kernel, dim3((s.n_buckets + 255) / 256, s.n_seg), dim3(256), 0, stream, counts, s,
                     totals);
  hipLaunchKernelGGL(sort_scan_buckets_kernel, dim3(s.n_seg), dim3(1024), 0, stream, totals, s);
  hipLaunchKernelGGL(sort_scatter_kernel, tg, dim3(64), lds, stream, buckets, s, counts, totals, perm, inv);
  return hipGetLastError();
}

}  // namespace rlsh
