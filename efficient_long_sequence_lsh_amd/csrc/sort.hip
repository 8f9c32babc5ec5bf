// Stage 2: stable sort of each (batch, head, round) segment by bucket id.
//
// "Reformer: The Efficient Transformer" (research summary), Summary: positions
// are sorted by bucket so that similar vectors become neighbours; Key points,
// LSH attention bullet: chunks are cut from the sorted order.  Ties keep the
// original position order (stable), so the permutation is unique.
//
// Design for gfx950: bucket ids are small integers (< 2^14), so one counting
// pass replaces a comparison sort.  A segment is cut into tiles.
//   hist:    per-tile bucket counts with LDS atomics (order does not matter
//            here), layout [segment][tile][bucket]
//   scan:    one thread per (segment, bucket): exclusive prefix over tiles
//            (in place) and the bucket total; the exclusive prefix over
//            buckets of the totals (the bucket bases) is formed by each
//            scatter wavefront for its own segment
//   scatter: one wavefront per tile walks it in position order, 64 keys at a
//            time, with the keys of 32 groups loaded ahead.  Equal keys inside
//            a group are found through a representative lane per key (LDS
//            byte per bucket) and a 64-bit peer mask per representative, or
//            with one ballot per key bit when the LDS would not hold the
//            representatives; each distinct key costs one LDS update by its
//            lowest lane and ranks come from a popcount.
//            slot = bucket base + earlier tiles + rank;
//            perm[slot] = position, inv[position] = slot.
// Workgroups of one segment are placed on one XCD (the hardware deals block
// b to XCD b % 8), so the scattered 4-byte writes of a segment meet in that
// XCD's L2 and leave it as whole lines.
// Keys outside [0, n_buckets) are clamped into the range.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace rlsh {

namespace {

constexpr int kHistThreads = 256;
constexpr int kHistUnroll = 8;
constexpr int kScanThreads = 256;
constexpr int kScanBatch = 32;
constexpr int kScatterBatch = 32;

__device__ __forceinline__ int clamp_key(int key, int n_buckets) { return min(max(key, 0), n_buckets - 1); }

// Tile (segment, tile index) of this workgroup under the XCD-aware order.
__device__ __forceinline__ bool tile_of_block(const SortShape& s, int per_xcd, int& seg, int& t) {
  const int b = blockIdx.x;
  const int logical = (b % 8) * per_xcd + b / 8;
  if (logical >= s.n_seg * s.n_tiles) return false;
  seg = logical / s.n_tiles;
  t = logical - seg * s.n_tiles;
  return true;
}

__device__ __forceinline__ uint64_t match_key(int key, bool active, int key_bits) {
  uint64_t peers = __ballot(active);
  for (int bit = 0; bit < key_bits; ++bit) {
    bool set = (key >> bit) & 1;
    uint64_t bal = __ballot(active && set);
    peers &= set ? bal : ~bal;
  }
  return peers;
}

__global__ __launch_bounds__(kHistThreads) void sort_hist_kernel(const int32_t* __restrict__ buckets, SortShape s,
                                                                 int per_xcd, int32_t* __restrict__ counts) {
  extern __shared__ int32_t cnt[];
  int seg, t;
  if (!tile_of_block(s, per_xcd, seg, t)) return;
  for (int k = threadIdx.x; k < s.n_buckets; k += kHistThreads) cnt[k] = 0;
  __syncthreads();
  const int32_t* keys = buckets + static_cast<size_t>(seg) * s.seq_len;
  const int p0 = t * s.tile, p1 = min(s.seq_len, p0 + s.tile);
  for (int base = p0; base < p1; base += kHistThreads * kHistUnroll) {
    int key[kHistUnroll];
#pragma unroll
    for (int i = 0; i < kHistUnroll; ++i)   // unconditional loads (clamped index) stay in flight together
      key[i] = keys[min(base + static_cast<int>(threadIdx.x) + kHistThreads * i, p1 - 1)];
#pragma unroll
    for (int i = 0; i < kHistUnroll; ++i)
      if (base + static_cast<int>(threadIdx.x) + kHistThreads * i < p1) atomicAdd(&cnt[clamp_key(key[i], s.n_buckets)], 1);
  }
  __syncthreads();
  int32_t* out = counts + (static_cast<size_t>(seg) * s.n_tiles + t) * s.n_buckets;
  for (int k = threadIdx.x; k < s.n_buckets; k += kHistThreads) out[k] = cnt[k];
}

// grid (n_seg, ceil(n_buckets / 256)): thread = one bucket of one segment.
// Exclusive prefix of its count over tiles, in place, and its total.
__global__ __launch_bounds__(kScanThreads) void sort_scan_kernel(int32_t* __restrict__ counts, SortShape s,
                                                                 int32_t* __restrict__ bucket_total) {
  const int seg = blockIdx.x;
  const int k = blockIdx.y * kScanThreads + threadIdx.x;
  if (k >= s.n_buckets) return;
  int32_t* c = counts + static_cast<size_t>(seg) * s.n_tiles * s.n_buckets + k;
  int run = 0;
  for (int t0 = 0; t0 < s.n_tiles; t0 += kScanBatch) {
    int v[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)   // unconditional loads (clamped index) stay in flight together
      v[i] = c[static_cast<size_t>(min(t0 + i, s.n_tiles - 1)) * s.n_buckets];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (t0 + i < s.n_tiles) {
        c[static_cast<size_t>(t0 + i) * s.n_buckets] = run;
        run += v[i];
      }
  }
  bucket_total[static_cast<size_t>(seg) * s.n_buckets + k] = run;
}

// LDS bytes of the scatter kernel: cur[n_buckets] (int32), then for the
// representative-lane ranking rep[n_buckets] (one byte each) and 64 peer masks.
__host__ __device__ constexpr size_t scatter_rep_offset(int n_buckets) { return static_cast<size_t>(n_buckets) * 4; }
__host__ __device__ constexpr size_t scatter_mask_offset(int n_buckets) {
  return align_up(scatter_rep_offset(n_buckets) + static_cast<size_t>(n_buckets), 8);
}
__host__ __device__ constexpr size_t scatter_lds_bytes(int n_buckets, bool reps) {
  return reps ? scatter_mask_offset(n_buckets) + 64 * sizeof(uint64_t) : scatter_rep_offset(n_buckets);
}

// Peers of this lane (lanes of the group holding the same key).  With REPS,
// every active lane writes its lane id to rep[key]; one write per key
// survives, so all lanes of a key read back the same representative lane and
// lanes of different keys read different ones.  Each lane then sets its bit
// in the 64-bit mask of its representative and reads the mask back.  A
// wavefront's LDS instructions complete in order, so each read sees the whole
// group's writes; relaxed atomics keep the compiler from forwarding a lane's
// own store to its load.  The caller clears the mask (leader lane) after use.
// Without REPS, one ballot per key bit.
template <bool REPS>
__device__ __forceinline__ uint64_t group_peers(int key, bool act, int lane, int key_bits, uint8_t* rep,
                                                uint64_t* mask, int& r) {
  if (!REPS) return match_key(key, act, key_bits);
  if (act) __hip_atomic_store(&rep[key], static_cast<uint8_t>(lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  r = act ? static_cast<int>(__hip_atomic_load(&rep[key], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) : 0;
  if (act) __hip_atomic_fetch_or(&mask[r], 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return act ? __hip_atomic_load(&mask[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0ull;
}

template <bool REPS>
__global__ __launch_bounds__(64) void sort_scatter_kernel(const int32_t* __restrict__ buckets, SortShape s,
                                                          int per_xcd, const int32_t* __restrict__ tile_off,
                                                          const int32_t* __restrict__ bucket_total,
                                                          int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  extern __shared__ __align__(16) unsigned char sort_lds[];
  int32_t* cur = reinterpret_cast<int32_t*>(sort_lds);
  uint8_t* rep = sort_lds + scatter_rep_offset(s.n_buckets);
  uint64_t* mask = reinterpret_cast<uint64_t*>(sort_lds + scatter_mask_offset(s.n_buckets));
  int seg, t;
  if (!tile_of_block(s, per_xcd, seg, t)) return;
  const int lane = threadIdx.x;
  const int32_t* off = tile_off + (static_cast<size_t>(seg) * s.n_tiles + t) * s.n_buckets;
  // Bucket bases of this segment (exclusive prefix of the totals over
  // buckets): lane owns the contiguous buckets [lane*per, lane*per + per).
  // cur[k] = base of k + this tile's offset in bucket k.
  const int32_t* tot = bucket_total + static_cast<size_t>(seg) * s.n_buckets;
  const int per = (s.n_buckets + 63) / 64;
  const int k0 = min(s.n_buckets, lane * per), k1 = min(s.n_buckets, k0 + per);
  int mine = 0;
  for (int kb = k0; kb < k1; kb += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = tot[min(kb + i, s.n_buckets - 1)];   // in flight together
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (kb + i < k1) mine += v[i];
  }
  int inc = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  int run = inc - mine;
  for (int kb = k0; kb < k1; kb += 8) {
    int v[8], o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = min(kb + i, s.n_buckets - 1);
      v[i] = tot[k];
      o[i] = off[k];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (kb + i < k1) {
        cur[kb + i] = run + o[i];
        run += v[i];
      }
  }
  if (REPS) mask[lane] = 0ull;
  __syncthreads();
  const size_t seg_base = static_cast<size_t>(seg) * s.seq_len;
  const int32_t* keys = buckets + seg_base;
  const int p0 = t * s.tile, p1 = min(s.seq_len, p0 + s.tile);
  const uint64_t lower_lanes = (1ull << lane) - 1ull;
  for (int base = p0; base < p1; base += 64 * kScatterBatch) {
    int key[kScatterBatch];
#pragma unroll
    for (int i = 0; i < kScatterBatch; ++i)   // unconditional loads (clamped index) stay in flight together
      key[i] = keys[min(base + 64 * i + lane, p1 - 1)];
    // Wait for every key before the first store: the store counter shares
    // vmcnt with the loads, and per-group waits would otherwise also wait for
    // the scattered stores of earlier groups.
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int i = 0; i < kScatterBatch; ++i) key[i] = clamp_key(key[i], s.n_buckets);
#pragma unroll
    for (int i = 0; i < kScatterBatch; ++i) {
      const int pos = base + 64 * i + lane;
      const bool act = pos < p1;
      int r = 0;
      const uint64_t peers = group_peers<REPS>(key[i], act, lane, s.key_bits, rep, mask, r);
      const int rank = __popcll(peers & lower_lanes);
      const int start = act ? cur[key[i]] : 0;
      if (act && rank == 0) {
        cur[key[i]] = start + __popcll(peers);
        if (REPS) __hip_atomic_store(&mask[r], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (act) {
        const int slot = start + rank;
        perm[seg_base + slot] = pos;
        if (inv != nullptr) inv[seg_base + pos] = slot;
      }
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
  int32_t* totals = reinterpret_cast<int32_t*>(   // bucket totals [seg][bucket]
      ws + align_up(static_cast<size_t>(s.n_seg) * s.n_tiles * s.n_buckets * sizeof(int32_t), 256));
  const size_t lds = static_cast<size_t>(s.n_buckets) * sizeof(int32_t);
  const int n_blocks = s.n_seg * s.n_tiles;
  const int per_xcd = (n_blocks + 7) / 8;
  hipLaunchKernelGGL(sort_hist_kernel, dim3(8 * per_xcd), dim3(kHistThreads), lds, stream, buckets, s, per_xcd,
                     counts);
  hipLaunchKernelGGL(sort_scan_kernel, dim3(s.n_seg, (s.n_buckets + kScanThreads - 1) / kScanThreads),
                     dim3(kScanThreads), 0, stream, counts, s, totals);
  const size_t rep_lds = scatter_lds_bytes(s.n_buckets, true);
  if (rep_lds <= 65536)
    hipLaunchKernelGGL(sort_scatter_kernel<true>, dim3(8 * per_xcd), dim3(64), rep_lds, stream, buckets, s, per_xcd,
                       counts, totals, perm, inv);
  else
    hipLaunchKernelGGL(sort_scatter_kernel<false>, dim3(8 * per_xcd), dim3(64), scatter_lds_bytes(s.n_buckets, false),
                       stream, buckets, s, per_xcd, counts, totals, perm, inv);
  return hipGetLastError();
}

}  // namespace rlsh
