// Stage 2: stable sort of each (batch, head, round) segment by bucket id.
//
// "Reformer: The Efficient Transformer" (research summary), Summary: positions
// are sorted by bucket so that similar vectors become neighbours; Key points,
// LSH attention bullet: chunks are cut from the sorted order.  Ties keep the
// original position order (stable), so the permutation is unique.
//
// Design for gfx950: bucket ids are small integers (< 2^14), so counting
// passes replace a comparison sort.  Every pass ranks its items the same way:
// each wavefront takes a contiguous run of items and walks it 64 at a time;
// the lanes holding the same key are found with one ballot per key bit, and
// rank = the wavefront's running count of the key (a per-wavefront LDS table)
// + the lower lanes holding it.  After a barrier, the counts of the earlier
// wavefronts and the keys before are added from the tables.
//
// Three shapes of the work:
//   block:   a segment of at most 12288 positions with at most 256 buckets is
//            sorted by one workgroup of sixteen wavefronts, the permutation
//            assembled in LDS and written out contiguously (one kernel).
//   tiles:   otherwise the segment is cut into tiles of 4096 positions, one
//            workgroup of four wavefronts each.
//              hist:    per-tile bin counts (LDS atomics), [segment][tile][bin]
//              scan:    one thread per (segment, bin): exclusive prefix over
//                       tiles (in place) and the bin total
//              scatter: the tile is ranked and ordered by bin in LDS, then
//                       written out bin run by bin run: slot = bin base (the
//                       prefix of the totals over bins) + earlier tiles + rank.
//            One pass (bin = bucket) for up to 1024 buckets when a segment's
//            slots fit in its XCD's L2 (at most 131072 positions) or for up to
//            64 buckets.
//   two passes: the tile scatter partitions by the top six bucket bits into a
//            temporary array of (low bucket bits, position) entries, and the
//            block kernel sorts each (segment, coarse bin) range of entries by
//            the low bits into its own contiguous range of the permutation (a
//            range above 12288 entries is counted first and ranked in chunks
//            written in place).
// Workgroups of one segment's tiles are placed on one XCD (the hardware deals
// block b to XCD b % 8), so their writes meet in that XCD's L2.
// Keys outside [0, n_buckets) are clamped into the range.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>
#include <type_traits>

namespace rlsh {

namespace {

constexpr int kThreads = 256;                 // tile workgroups
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 4096;                   // positions per tile
constexpr int kGroups = kTile / kThreads;     // groups of 64 items per wavefront and tile
constexpr int kScanThreads = 64;
constexpr int kScanBatch = 32;
constexpr int kCoarseBits = 6;                // bins of the first of two passes
constexpr int kOnePassMaxBits = 10;           // one tile pass for up to 1024 buckets ...
constexpr int kOnePassMaxLen = 131072;        // ... and segments of up to 512 KB of slots
constexpr int kMaxBinsPerThread = (1 << kOnePassMaxBits) / kThreads;
constexpr int kBlkThreads = 1024;             // block workgroups
constexpr int kBlkWaves = kBlkThreads / kWave;
constexpr int kBlkGroups = 12;                // groups of 64 items per wavefront at most
constexpr int kBlkItems = kBlkWaves * kBlkGroups * kWave;   // 12288
constexpr int kBlkBits = 8;
constexpr int kBlkBins = 1 << kBlkBits;
static_assert(kMaxSortKeyBits - kCoarseBits <= kBlkBits, "the low bits of two passes fit the block kernel");

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

// Lanes of this wavefront whose active flag is set and whose key equals this
// lane's.  Keys are below 2^BITS, so higher bits need no ballot.  Per bit: the
// ballot of the lanes that have it set, kept where this lane has it set too,
// complemented where it does not.
template <int BITS>
__device__ __forceinline__ uint64_t match_key(int key, bool active) {
  const uint64_t act = __builtin_amdgcn_ballot_w64(active);
  uint32_t lo = static_cast<uint32_t>(act), hi = static_cast<uint32_t>(act >> 32);
#pragma unroll
  for (int bit = 0; bit < BITS; ++bit) {
    const uint32_t all = static_cast<uint32_t>(__builtin_amdgcn_sbfe(key, bit, 1));   // 0 or all ones
    const uint64_t bal = __builtin_amdgcn_ballot_w64(all != 0u);
    lo &= ~(static_cast<uint32_t>(bal) ^ all);
    hi &= ~(static_cast<uint32_t>(bal >> 32) ^ all);
  }
  return static_cast<uint64_t>(hi) << 32 | lo;
}

// Exclusive prefix of v over the workgroup's threads in thread order; the
// workgroup total in `total`.  Contains two barriers.
template <int WAVES>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform, known to the compiler
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) {
    const int x = wsum[i];
    if (i < w) before += x;
    total += x;
  }
  __syncthreads();
  return before + inc - v;
}

// Stable ranking inside one wavefront of up to G groups of 64 items, in item
// order (group g = the wavefront's items g*64 + lane; n_act of them exist).
// kr[g] holds the item's key on entry and (key << 16 | rank) on return, rank =
// items of the same key earlier in the wavefront's run (< 2^16).  lc is this
// wavefront's table of running counts per key, zero on entry and the
// wavefront's count of each key on return.  Per group all active lanes read
// their key's count and the lowest lane of each key writes it back advanced
// by the group's count; a wavefront's LDS instructions complete in order, so
// the next group reads the advanced counts.  Relaxed atomics keep the
// compiler from forwarding a lane's own store to a later load.
template <int BITS, int G>
__device__ __forceinline__ void wave_rank(int (&kr)[G], int n_act, int* lc) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t lower = (1ull << lane) - 1ull;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g * kWave >= n_act) break;   // uniform over the wavefront
    const bool act = g * kWave + lane < n_act;
    const int key = kr[g];
    const uint64_t peers = match_key<BITS>(key, act);
    const int before = act ? __hip_atomic_load(&lc[key], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0;
    kr[g] = key << 16 | (before + __popcll(peers & lower));
    if (act && (peers & lower) == 0ull)
      __hip_atomic_store(&lc[key], before + __popcll(peers), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// For keys [k0, k1) owned by this thread: lc[v][k] (v < WAVES, row stride
// `stride`) becomes the exclusive prefix over wavefronts, and tot[j] the sum.
template <int WAVES, int PER>
__device__ __forceinline__ void scan_over_waves(int* lc, int stride, int k0, int k1, int (&tot)[PER]) {
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    tot[j] = 0;
    if (k0 + j >= k1) continue;
    int x[WAVES];
#pragma unroll
    for (int v = 0; v < WAVES; ++v) x[v] = lc[v * stride + k0 + j];   // read together
    int run = 0;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
      lc[v * stride + k0 + j] = run;
      run += x[v];
    }
    tot[j] = run;
  }
}

__global__ __launch_bounds__(kThreads) void sort_hist_kernel(const int32_t* __restrict__ buckets, SortShape s,
                                                             int per_xcd, int32_t* __restrict__ counts) {
  extern __shared__ int32_t cnt[];
  int seg, t;
  if (!tile_of_block(s, per_xcd, seg, t)) return;
  for (int k = threadIdx.x; k < s.n_bins; k += kThreads) cnt[k] = 0;
  const int p0 = t * kTile;
  const int n_here = min(kTile, s.seq_len - p0);
  const int32_t* keys = buckets + static_cast<size_t>(seg) * s.seq_len + p0;
  int key[kGroups];
#pragma unroll
  for (int i = 0; i < kGroups; ++i)   // unconditional loads (clamped index) stay in flight together
    key[i] = keys[min(i * kThreads + static_cast<int>(threadIdx.x), n_here - 1)];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kGroups; ++i)
    if (i * kThreads + static_cast<int>(threadIdx.x) < n_here)
      atomicAdd(&cnt[clamp_key(key[i], s.n_buckets) >> s.bin_shift], 1);
  __syncthreads();
  int32_t* out = counts + (static_cast<size_t>(seg) * s.n_tiles + t) * s.n_bins;
  for (int k = threadIdx.x; k < s.n_bins; k += kThreads) out[k] = cnt[k];
}

// grid (n_seg, ceil(n_bins / 64)): thread = one bin of one segment.
// Exclusive prefix of its count over tiles, in place, and its total.
__global__ __launch_bounds__(kScanThreads) void sort_scan_kernel(int32_t* __restrict__ counts, SortShape s,
                                                                 int32_t* __restrict__ bin_total) {
  const int seg = blockIdx.x;
  const int k = blockIdx.y * kScanThreads + threadIdx.x;
  if (k >= s.n_bins) return;
  int32_t* c = counts + static_cast<size_t>(seg) * s.n_tiles * s.n_bins + k;
  int run = 0;
  for (int t0 = 0; t0 < s.n_tiles; t0 += kScanBatch) {
    int v[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)   // unconditional loads (clamped index) stay in flight together
      v[i] = c[static_cast<size_t>(min(t0 + i, s.n_tiles - 1)) * s.n_bins];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (t0 + i < s.n_tiles) {
        c[static_cast<size_t>(t0 + i) * s.n_bins] = run;
        run += v[i];
      }
  }
  bin_total[static_cast<size_t>(seg) * s.n_bins + k] = run;
}

// Where the tile scatter writes: the permutation itself (one pass), or the
// entries of the second pass, (low bits << pos_bits | position) in 32 bits or
// (low bits << 32 | position) in 64 bits.
enum ScatterOut { kToPerm = 0, kToEntries32 = 1, kToEntries64 = 2 };

// LDS of the tile scatter: the staged values [kTile] (4 or 8 bytes), cur and
// lbase [n_bins], lc [kWaves][n_bins] and the staged values' bins [kTile]
// (2 bytes).
__host__ __device__ constexpr size_t scatter_lds_bytes(int n_bins, bool wide) {
  return static_cast<size_t>(kTile) * (wide ? 8 : 4) + static_cast<size_t>(2 + kWaves) * n_bins * 4 +
         static_cast<size_t>(kTile) * 2;
}

template <int OUT, int BITS>
__global__ __launch_bounds__(kThreads) void sort_scatter_kernel(const int32_t* __restrict__ buckets, SortShape s,
                                                                int per_xcd, const int32_t* __restrict__ tile_off,
                                                                const int32_t* __restrict__ totals,
                                                                void* __restrict__ dst, int32_t* __restrict__ inv) {
  typedef typename std::conditional<OUT == kToEntries64, uint64_t, uint32_t>::type value_t;
  extern __shared__ __align__(16) int32_t sort_lds[];
  __shared__ int wsum[kWaves];
  value_t* stage = reinterpret_cast<value_t*>(sort_lds);                       // [kTile]
  int32_t* cur = reinterpret_cast<int32_t*>(stage + kTile);                     // [n_bins]
  int32_t* lbase = cur + s.n_bins;                                              // [n_bins]
  int32_t* lc = lbase + s.n_bins;                                               // [kWaves][n_bins]
  uint16_t* stage_bin = reinterpret_cast<uint16_t*>(lc + kWaves * s.n_bins);   // [kTile]
  int seg, t;
  if (!tile_of_block(s, per_xcd, seg, t)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform, known to the compiler
  const size_t seg_base = static_cast<size_t>(seg) * s.seq_len;
  const int p0 = t * kTile;
  const int n_here = min(kTile, s.seq_len - p0);
  // Wavefront w ranks the tile's items [w * kWaveItems, (w + 1) * kWaveItems).
  constexpr int kWaveItems = kGroups * kWave;
  const int q0 = w * kWaveItems;
  const int n_act = n_here - q0;   // items of this wavefront (may be <= 0)
  const int32_t* keys = buckets + seg_base + p0;
  int key[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g)   // in flight while the bases are formed
    key[g] = keys[min(q0 + g * kWave + lane, n_here - 1)];

  // cur[b] = base of bin b in the segment (prefix of the totals over bins,
  // each thread owning a contiguous run of bins) + this tile's offset in b.
  const int32_t* tot = totals + static_cast<size_t>(seg) * s.n_bins;
  const int32_t* off = tile_off + (static_cast<size_t>(seg) * s.n_tiles + t) * s.n_bins;
  const int per = (s.n_bins + kThreads - 1) / kThreads;   // <= kMaxBinsPerThread
  const int b0 = min(s.n_bins, static_cast<int>(threadIdx.x) * per), b1 = min(s.n_bins, b0 + per);
  int tv[kMaxBinsPerThread], ov[kMaxBinsPerThread];
#pragma unroll
  for (int j = 0; j < kMaxBinsPerThread; ++j) {   // in flight together
    const int b = min(b0 + j, s.n_bins - 1);
    tv[j] = tot[b];
    ov[j] = off[b];
  }
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kMaxBinsPerThread; ++j)
    if (b0 + j < b1) mine += tv[j];
  int total;
  int run = block_exclusive_scan<kWaves>(mine, wsum, total);
#pragma unroll
  for (int j = 0; j < kMaxBinsPerThread; ++j)
    if (b0 + j < b1) {
      cur[b0 + j] = run + ov[j];
      run += tv[j];
    }
  int* my_lc = lc + w * s.n_bins;
  for (int b = lane; b < s.n_bins; b += kWave) my_lc[b] = 0;

  const uint32_t low_mask = (1u << s.bin_shift) - 1u;
  int kr[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    key[g] = clamp_key(key[g], s.n_buckets);
    kr[g] = key[g] >> s.bin_shift;
  }
  wave_rank<BITS, kGroups>(kr, n_act, my_lc);
  __syncthreads();   // every wavefront's counts are complete

  // Order the tile by bin in LDS: lbase[b] = the tile's items of bins below b.
  int cnt[kMaxBinsPerThread];
  scan_over_waves<kWaves, kMaxBinsPerThread>(lc, s.n_bins, b0, b1, cnt);
  int lmine = 0;
#pragma unroll
  for (int j = 0; j < kMaxBinsPerThread; ++j) lmine += cnt[j];
  int lrun = block_exclusive_scan<kWaves>(lmine, wsum, total);
#pragma unroll
  for (int j = 0; j < kMaxBinsPerThread; ++j)
    if (b0 + j < b1) {
      lbase[b0 + j] = lrun;
      lrun += cnt[j];
    }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (g * kWave >= n_act) break;   // uniform over the wavefront
    const int i = g * kWave + lane;
    if (i >= n_act) continue;
    const int b = kr[g] >> 16;
    // The clamp is a guard only: the ranking keeps local slots inside the tile.
    const int local = min(max(lbase[b] + lc[w * s.n_bins + b] + (kr[g] & 0xffff), 0), kTile - 1);
    const uint32_t pos = static_cast<uint32_t>(p0 + q0 + i);
    value_t v;
    if (OUT == kToPerm) v = pos;
    else if (OUT == kToEntries32) v = (static_cast<uint32_t>(key[g]) & low_mask) << s.pos_bits | pos;
    else v = static_cast<value_t>(static_cast<uint32_t>(key[g]) & low_mask) << 32 | pos;
    stage[local] = v;
    stage_bin[local] = static_cast<uint16_t>(b);
  }
  __syncthreads();
  // Bin runs out: consecutive local slots of one bin go to consecutive slots.
#pragma unroll 4
  for (int j = threadIdx.x; j < n_here; j += kThreads) {
    const int b = stage_bin[j];
    const int slot = min(max(cur[b] + j - lbase[b], 0), s.seq_len - 1);   // clamp: guard only
    static_cast<value_t*>(dst)[seg_base + slot] = stage[j];
    if (OUT == kToPerm && inv != nullptr) inv[seg_base + static_cast<int>(stage[j])] = slot;
  }
}

// The block kernel's sources: bucket ids of a whole segment, or the entries of
// one (segment, coarse bin) range of the two-pass temporary array.
enum BlockSrc { kFromBuckets = 0, kFromEntries32 = 1, kFromEntries64 = 2 };

// Stable counting sort of a range of at most kBlkItems items held in LDS, or,
// for a longer range of entries, the same ranking in chunks after a count of
// the whole range, each chunk written straight to its slots.
template <int SRC, int BITS>
__global__ __launch_bounds__(kBlkThreads) void sort_block_kernel(const void* __restrict__ src, SortShape s,
                                                                 const int32_t* __restrict__ totals,
                                                                 int32_t* __restrict__ perm,
                                                                 int32_t* __restrict__ inv) {
  typedef typename std::conditional<SRC == kFromEntries64, uint64_t, uint32_t>::type item_t;
  __shared__ int32_t stage[kBlkItems];
  __shared__ int32_t lc[kBlkWaves * kBlkBins];
  __shared__ int32_t kbase[kBlkBins];
  __shared__ int wsum[kBlkWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform, known to the compiler
  const int tid = threadIdx.x;
  int seg, first, n, nk;   // items [first, first + n) of the segment; keys below nk
  if (SRC == kFromBuckets) {
    seg = blockIdx.x;
    first = 0;
    n = s.seq_len;
    nk = s.n_buckets;
  } else {
    seg = blockIdx.x / s.n_bins;
    const int c = blockIdx.x - seg * s.n_bins;
    const int32_t* tot = totals + static_cast<size_t>(seg) * s.n_bins;
    block_exclusive_scan<kBlkWaves>(tid < c ? tot[tid] : 0, wsum, first);   // entries of the bins before c
    n = tot[c];
    nk = 1 << s.bin_shift;
  }
  if (n == 0) return;   // uniform over the workgroup
  const size_t seg_base = static_cast<size_t>(seg) * s.seq_len;
  const item_t* items = static_cast<const item_t*>(src) + seg_base + first;
  const uint32_t pos_mask = SRC == kFromEntries32 ? (1u << s.pos_bits) - 1u : ~0u;
  const int key_shift = SRC == kFromEntries64 ? 32 : s.pos_bits;
  // Key and position of an item (masks and clamps are guards only: the first
  // pass writes every entry of the range with a position inside the segment).
  auto key_of = [&](item_t it) {
    return SRC == kFromBuckets ? clamp_key(static_cast<int>(it), nk) : static_cast<int>(it >> key_shift) & (nk - 1);
  };
  auto pos_of = [&](item_t it) { return min(static_cast<int>(static_cast<uint32_t>(it) & pos_mask), s.seq_len - 1); };
  const bool resident = n <= kBlkItems;   // uniform over the workgroup
  const int kk0 = min(nk, tid), kk1 = min(nk, tid + 1);   // key owned by this thread in the scans
  if (!resident) {
    // Count the whole range: kbase[k] = first slot of key k in the segment.
    if (tid < nk) kbase[tid] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += kBlkThreads * 8) {
      item_t e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) e[u] = items[min(i0 + u * kBlkThreads + tid, n - 1)];   // in flight together
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * kBlkThreads + tid < n) atomicAdd(&kbase[key_of(e[u])], 1);
    }
    __syncthreads();
    int unused;
    const int c = tid < nk ? kbase[tid] : 0;
    const int ex = block_exclusive_scan<kBlkWaves>(c, wsum, unused);
    if (tid < nk) kbase[tid] = first + ex;
  }
  int* my_lc = lc + w * kBlkBins;
  for (int i0 = 0; i0 < n; i0 += kBlkItems) {
    const int m = min(kBlkItems, n - i0);
    const int per_wave = (m + kBlkWaves * kWave - 1) / (kBlkWaves * kWave) * kWave;
    const int q0 = w * per_wave;
    const int n_act = min(per_wave, m - q0);   // may be <= 0
    // Positions are kept only for entries; a segment's item i is position i.
    int kr[kBlkGroups], pos[SRC == kFromBuckets ? 1 : kBlkGroups];
    item_t it[kBlkGroups];
    // Unconditional loads (index clamped into the chunk) in flight together,
    // addressed as a uniform base plus a 32-bit byte offset per lane (fewer
    // registers than one 64-bit address per load).
    const char* chunk = reinterpret_cast<const char*>(items + i0);
#pragma unroll
    for (int g = 0; g < kBlkGroups; ++g)
      it[g] = *reinterpret_cast<const item_t*>(
          chunk + static_cast<uint32_t>(min(q0 + g * kWave + lane, m - 1)) * static_cast<uint32_t>(sizeof(item_t)));
#pragma unroll
    for (int g = 0; g < kBlkGroups; ++g) {
      kr[g] = key_of(it[g]);
      if constexpr (SRC != kFromBuckets) pos[g] = pos_of(it[g]);
    }
    for (int k = lane; k < nk; k += kWave) my_lc[k] = 0;
    wave_rank<BITS, kBlkGroups>(kr, n_act, my_lc);
    __syncthreads();   // every wavefront's counts are complete
    int cnt[1];
    scan_over_waves<kBlkWaves, 1>(lc, kBlkBins, kk0, kk1, cnt);
    if (resident) {
      int unused;
      const int ex = block_exclusive_scan<kBlkWaves>(cnt[0], wsum, unused);
      if (tid < nk) kbase[tid] = ex;   // local slot of key tid's first item
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kBlkGroups; ++g) {
      if (g * kWave >= n_act) break;   // uniform over the wavefront
      if (g * kWave + lane >= n_act) continue;
      const int k = kr[g] >> 16;
      const int r = kbase[k] + lc[w * kBlkBins + k] + (kr[g] & 0xffff);
      int p;
      if constexpr (SRC == kFromBuckets) p = i0 + q0 + g * kWave + lane;
      else p = pos[g];
      if (resident) {
        const int local = min(max(r, 0), kBlkItems - 1);   // clamp: guard only
        stage[local] = p;
        if (inv != nullptr) inv[seg_base + p] = first + local;
      } else {
        const int slot = min(max(r, 0), s.seq_len - 1);   // clamp: guard only
        perm[seg_base + slot] = p;
        if (inv != nullptr) inv[seg_base + p] = slot;
      }
    }
    __syncthreads();   // the staged slots, or every read of kbase and the counts, are done
    if (resident) {
      for (int i = tid; i < n; i += kBlkThreads) perm[seg_base + first + i] = stage[i];
    } else {
      if (tid < nk) kbase[tid] += cnt[0];
      __syncthreads();   // kbase advanced before the counts are cleared again
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

int bits_for(long long n) {   // smallest b with 2^b >= n
  int b = 0;
  while ((1LL << b) < n) ++b;
  return b;
}

}  // namespace

SortShape make_sort_shape(int n_seg, int seq_len, int n_buckets) {
  SortShape s{};
  s.n_seg = n_seg;
  s.seq_len = seq_len;
  s.n_buckets = n_buckets;
  s.n_tiles = (seq_len + kTile - 1) / kTile;
  s.key_bits = bits_for(n_buckets);
  s.block = s.key_bits <= kBlkBits && seq_len <= kBlkItems;
  s.two_pass = !s.block && s.key_bits > kCoarseBits && (s.key_bits > kOnePassMaxBits || seq_len > kOnePassMaxLen);
  if (!s.two_pass) {
    s.n_bins = n_buckets;
    s.bin_bits = s.key_bits;
    s.bin_shift = 0;
  } else {
    s.bin_shift = s.key_bits - kCoarseBits;
    s.bin_bits = kCoarseBits;
    s.n_bins = ((n_buckets - 1) >> s.bin_shift) + 1;
    s.pos_bits = std::max(1, bits_for(seq_len));
    s.wide_entries = s.bin_shift + s.pos_bits > 32;
  }
  return s;
}

namespace {
struct SortScratch {
  size_t counts, totals, entries, total;
};
SortScratch sort_scratch(const SortShape& s) {
  SortScratch r{};
  if (s.block) return r;
  r.counts = align_up(static_cast<size_t>(s.n_seg) * s.n_tiles * s.n_bins * sizeof(int32_t), 256);
  r.totals = align_up(static_cast<size_t>(s.n_seg) * s.n_bins * sizeof(int32_t), 256);
  if (s.two_pass)
    r.entries = align_up(static_cast<size_t>(s.n_seg) * s.seq_len * (s.wide_entries ? 8 : 4), 256);
  r.total = r.counts + r.totals + r.entries;
  return r;
}
}  // namespace

size_t sort_scratch_bytes(const SortShape& s) {
  if (s.n_buckets <= 1) return 0;
  return sort_scratch(s).total;
}

hipError_t launch_sort(const int32_t* buckets, const SortShape& s, int32_t* perm, int32_t* inv, void* workspace,
                       hipStream_t stream) {
  if (s.n_buckets <= 1) {
    size_t n = static_cast<size_t>(s.n_seg) * s.seq_len;
    unsigned grid = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 8192));
    hipLaunchKernelGGL(iota_kernel, dim3(std::max(grid, 1u)), dim3(256), 0, stream, perm, inv, s.n_seg, s.seq_len);
    return hipGetLastError();
  }
  if (s.key_bits > kMaxSortKeyBits || s.n_bins > (1 << kOnePassMaxBits)) return hipErrorInvalidValue;
  const dim3 blk(kBlkThreads);
  if (s.block) {
    const void* src = buckets;
    if (s.key_bits <= 4)
      hipLaunchKernelGGL((sort_block_kernel<kFromBuckets, 4>), dim3(s.n_seg), blk, 0, stream, src, s, nullptr, perm,
                         inv);
    else
      hipLaunchKernelGGL((sort_block_kernel<kFromBuckets, kBlkBits>), dim3(s.n_seg), blk, 0, stream, src, s, nullptr,
                         perm, inv);
    return hipGetLastError();
  }
  const SortScratch sc = sort_scratch(s);
  char* ws = static_cast<char*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  int32_t* totals = reinterpret_cast<int32_t*>(ws + sc.counts);
  void* entries = ws + sc.counts + sc.totals;
  const int n_blocks = s.n_seg * s.n_tiles;
  const int per_xcd = (n_blocks + 7) / 8;
  const size_t hist_lds = static_cast<size_t>(s.n_bins) * sizeof(int32_t);
  hipLaunchKernelGGL(sort_hist_kernel, dim3(8 * per_xcd), dim3(kThreads), hist_lds, stream, buckets, s, per_xcd,
                     counts);
  hipLaunchKernelGGL(sort_scan_kernel, dim3(s.n_seg, (s.n_bins + kScanThreads - 1) / kScanThreads),
                     dim3(kScanThreads), 0, stream, counts, s, totals);
  const dim3 tiles(8 * per_xcd), block(kThreads);
  if (!s.two_pass) {
    void* out = perm;
    const size_t lds = scatter_lds_bytes(s.n_bins, false);
    if (s.bin_bits <= 6)
      hipLaunchKernelGGL((sort_scatter_kernel<kToPerm, 6>), tiles, block, lds, stream, buckets, s, per_xcd, counts,
                         totals, out, inv);
    else if (s.bin_bits <= 8)
      hipLaunchKernelGGL((sort_scatter_kernel<kToPerm, 8>), tiles, block, lds, stream, buckets, s, per_xcd, counts,
                         totals, out, inv);
    else
      hipLaunchKernelGGL((sort_scatter_kernel<kToPerm, kOnePassMaxBits>), tiles, block, lds, stream, buckets, s,
                         per_xcd, counts, totals, out, inv);
    return hipGetLastError();
  }
  const dim3 fine_grid(static_cast<unsigned>(s.n_seg) * static_cast<unsigned>(s.n_bins));
  const void* ent = entries;
  const bool few = s.bin_shift <= 4;   // low bits ranked by the second pass
  if (s.wide_entries) {
    hipLaunchKernelGGL((sort_scatter_kernel<kToEntries64, kCoarseBits>), tiles, block,
                       scatter_lds_bytes(s.n_bins, true), stream, buckets, s, per_xcd, counts, totals, entries,
                       nullptr);
    if (few)
      hipLaunchKernelGGL((sort_block_kernel<kFromEntries64, 4>), fine_grid, blk, 0, stream, ent, s, totals, perm, inv);
    else
      hipLaunchKernelGGL((sort_block_kernel<kFromEntries64, kBlkBits>), fine_grid, blk, 0, stream, ent, s, totals,
                         perm, inv);
  } else {
    hipLaunchKernelGGL((sort_scatter_kernel<kToEntries32, kCoarseBits>), tiles, block,
                       scatter_lds_bytes(s.n_bins, false), stream, buckets, s, per_xcd, counts, totals, entries,
                       nullptr);
    if (few)
      hipLaunchKernelGGL((sort_block_kernel<kFromEntries32, 4>), fine_grid, blk, 0, stream, ent, s, totals, perm, inv);
    else
      hipLaunchKernelGGL((sort_block_kernel<kFromEntries32, kBlkBits>), fine_grid, blk, 0, stream, ent, s, totals,
                         perm, inv);
  }
  return hipGetLastError();
}

}  // namespace rlsh
