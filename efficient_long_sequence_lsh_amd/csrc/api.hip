// C ABI of the LSH attention library: argument validation (pure host code,
// run before any HIP call), workspace carving and the launch sequence.
#include "reformer_lsh.h"

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <limits>
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

// Scratch of the allocation-free hash entry point: a file-scope device array
// (every GPU the library runs on holds its own copy until the process ends).
// Host code never passes this name to a kernel: it is a host-side stand-in.
// The device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[RLSH_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxBuckets = 16384;
constexpr int kMaxSegments = 65535;   // grid y-dimension bound for per-segment launches

thread_local char g_last_error[512] = "";

rlsh_status_t fail(rlsh_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

rlsh_status_t ok() {
  g_last_error[0] = '\0';
  return RLSH_OK;
}

rlsh_status_t hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(RLSH_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
  return ok();
}

// Shape checks shared by all entry points.  n_buckets < 0 means "not used".
rlsh_status_t check_shape(int batch, int heads, int seq_len, int d_head, int n_rounds, int n_buckets, int chunk_len) {
  if (batch < 1 || heads < 1 || seq_len < 1 || n_rounds < 1)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "batch, heads, seq_len and n_rounds must be >= 1 (got %d, %d, %d, %d)",
                batch, heads, seq_len, n_rounds);
  const long long total = static_cast<long long>(batch) * heads * n_rounds * seq_len;
  if (total >= (1LL << 31))
    return fail(RLSH_ERR_INVALID_ARGUMENT, "batch*heads*n_rounds*seq_len = %lld must be < 2^31", total);
  if (static_cast<long long>(batch) * heads * n_rounds > kMaxSegments)
    return fail(RLSH_ERR_UNSUPPORTED, "batch*heads*n_rounds must be <= %d", kMaxSegments);
  if (d_head >= 0 && d_head != 64 && d_head != 128)
    return fail(RLSH_ERR_UNSUPPORTED, "d_head must be 64 or 128 (got %d)", d_head);
  if (n_buckets >= 0) {
    if (n_buckets < 1 || (n_buckets != 1 && (n_buckets % 2) != 0))
      return fail(RLSH_ERR_INVALID_ARGUMENT, "n_buckets must be 1 or even (got %d)", n_buckets);
    if (n_buckets > kMaxBuckets)
      return fail(RLSH_ERR_UNSUPPORTED, "n_buckets must be <= %d (got %d)", kMaxBuckets, n_buckets);
  }
  if (chunk_len >= 0) {
    if (chunk_len < 1) return fail(RLSH_ERR_INVALID_ARGUMENT, "chunk_len must be >= 1 (got %d)", chunk_len);
    const int m = std::min(chunk_len, seq_len);
    if (seq_len % m != 0)
      return fail(RLSH_ERR_INVALID_ARGUMENT, "seq_len %d must be a multiple of chunk_len %d (or chunk_len >= seq_len)",
                  seq_len, chunk_len);
  }
  return ok();
}

// Rows are moved with 16-byte vector loads and stores.
rlsh_status_t check_aligned(const void* p, const char* name) {
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0u)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  return ok();
}

rlsh_status_t check_dtype(rlsh_dtype_t dtype) {
  if (dtype != RLSH_F32 && dtype != RLSH_BF16) return fail(RLSH_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  return ok();
}

size_t tokens(int batch, int heads, int seq_len) {
  return static_cast<size_t>(batch) * heads * seq_len;
}

size_t a256(size_t x) { return rlsh::align_up(x, 256); }

size_t hash_ws(int batch, int heads, int seq_len, int d_head, int n_rounds, int n_buckets) {
  if (n_buckets <= 1) return 0;
  return rlsh::hash_scratch(rlsh::make_hash_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets)).total;
}

size_t sort_ws(int batch, int heads, int seq_len, int n_rounds, int n_buckets) {
  return rlsh::sort_scratch_bytes(rlsh::make_sort_shape(batch * heads * n_rounds, seq_len, n_buckets));
}

// Per-round intermediates: float32 o and z, or (bf16 inputs with 64-slot
// chunks) float16 o scaled per row plus (z, k) float pairs.
struct RoundLayout {
  bool compact;
  size_t o_bytes, z_bytes;
};

RoundLayout round_layout(rlsh_dtype_t dtype, int batch, int heads, int seq_len, int d_head, int n_rounds,
                         int chunk_len) {
  const size_t n = tokens(batch, heads, seq_len) * n_rounds;
  RoundLayout r{};
  r.compact = rlsh::compact_rounds_supported(dtype == RLSH_BF16, seq_len, chunk_len);
  // compact rows: float16 at d = 64, 12-bit block floating point at d = 128
  r.o_bytes = a256(n * (r.compact ? (d_head == 128 ? 3 * d_head / 2 : 2 * d_head) : d_head * sizeof(float)));
  r.z_bytes = r.compact ? 0 : a256(n * sizeof(float));   // compact rows carry their own z
  return r;
}

size_t attend_ws(rlsh_dtype_t dtype, int batch, int heads, int seq_len, int d_head, int n_rounds, int chunk_len) {
  const RoundLayout r = round_layout(dtype, batch, heads, seq_len, d_head, n_rounds, chunk_len);
  return r.o_bytes + r.z_bytes;
}

// Full pipeline layout: buckets | perm | region (per-round o, aliased earlier
// by the hash and sort scratch, which are dead once attention starts) | z.
struct FullLayout {
  RoundLayout rounds;
  size_t buckets, perm, region, z, total;
};

FullLayout full_layout(rlsh_dtype_t dtype, int batch, int heads, int seq_len, int d_head, int n_rounds, int n_buckets,
                       int chunk_len) {
  const size_t n = tokens(batch, heads, seq_len) * n_rounds;
  FullLayout f{};
  f.rounds = round_layout(dtype, batch, heads, seq_len, d_head, n_rounds, chunk_len);
  f.buckets = 0;
  f.perm = a256(n * sizeof(int32_t));
  size_t region = f.rounds.o_bytes;
  region = std::max(region, a256(hash_ws(batch, heads, seq_len, d_head, n_rounds, n_buckets)));
  region = std::max(region, a256(sort_ws(batch, heads, seq_len, n_rounds, n_buckets)));
  f.region = f.perm + a256(n * sizeof(int32_t));
  f.z = f.region + region;
  f.total = f.z + f.rounds.z_bytes;
  return f;
}

// chunk attention + combine into `out`, with the intermediates at o_mem / z_mem.
// mark (optional): event recorded between the two kernels.
hipError_t run_attend(const void* qk, const void* v, rlsh_dtype_t dtype, const int32_t* perm, int bh, int seq_len,
                      int d_head, int n_rounds, int chunk_len, int causal, void* out, const RoundLayout& rl,
                      void* o_mem, void* z_mem, hipStream_t stream, hipEvent_t* mark = nullptr,
                      float* lse = nullptr) {
  const bool bf16 = dtype == RLSH_BF16;
  hipError_t e;
  if (rl.compact) {
    uint16_t* o16 = static_cast<uint16_t*>(o_mem);   // z and k ride in the rows (no z_mem)
    e = rlsh::launch_attend_combine_compact(qk, v, perm, bh, seq_len, d_head, n_rounds, causal != 0, o16, out, lse,
                                            stream, mark);
  } else {
    float* o = static_cast<float*>(o_mem);
    float* z = static_cast<float*>(z_mem);
    e = rlsh::launch_chunk_attend(qk, v, bf16, perm, bh, seq_len, d_head, n_rounds, chunk_len, causal != 0, o, z,
                                  stream);
    if (e == hipSuccess && mark) e = hipEventRecord(*mark, stream);
    if (e == hipSuccess) e = rlsh::launch_combine(o, z, v, bf16, bh, seq_len, d_head, n_rounds, out, lse, stream);
  }
  return e;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up on the first call per device
// (with that device current) and kept.
rlsh_status_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RLSH_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch is tracked for", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(RLSH_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" {

const char* reformer_lsh_status_string(rlsh_status_t status) {
  switch (status) {
    case RLSH_OK: return "RLSH_OK";
    case RLSH_ERR_INVALID_ARGUMENT: return "RLSH_ERR_INVALID_ARGUMENT";
    case RLSH_ERR_UNSUPPORTED: return "RLSH_ERR_UNSUPPORTED";
    case RLSH_ERR_WORKSPACE_TOO_SMALL: return "RLSH_ERR_WORKSPACE_TOO_SMALL";
    case RLSH_ERR_HIP: return "RLSH_ERR_HIP";
  }
  return "RLSH_UNKNOWN_STATUS";
}

const char* reformer_lsh_last_error(void) { return g_last_error; }

int reformer_lsh_version(void) { return 10000; }

size_t reformer_lsh_hash_workspace_bytes(int batch, int heads, int seq_len, int d_head, int n_rounds, int n_buckets) {
  if (check_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets, -1) != RLSH_OK) return 0;
  return hash_ws(batch, heads, seq_len, d_head, n_rounds, n_buckets);
}

rlsh_status_t reformer_lsh_hash(const void* qk, rlsh_dtype_t dtype, const float* rotations, int batch, int heads,
                                int seq_len, int d_head, int n_rounds, int n_buckets, int32_t* buckets,
                                int32_t* n_near_ties, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets, -1);
  if (st != RLSH_OK) return st;
  if ((st = check_dtype(dtype)) != RLSH_OK) return st;
  if (qk == nullptr || buckets == nullptr) return fail(RLSH_ERR_INVALID_ARGUMENT, "qk and buckets must be non-null");
  if ((st = check_aligned(qk, "qk")) != RLSH_OK) return st;
  if ((st = check_aligned(workspace, "workspace")) != RLSH_OK) return st;
  const size_t need = hash_ws(batch, heads, seq_len, d_head, n_rounds, n_buckets);
  if (n_buckets > 1) {
    if (rotations == nullptr) return fail(RLSH_ERR_INVALID_ARGUMENT, "rotations must be non-null when n_buckets > 1");
    if (workspace == nullptr || workspace_bytes < need)
      return fail(RLSH_ERR_WORKSPACE_TOO_SMALL, "hash workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  }
  const size_t n = tokens(batch, heads, seq_len) * n_rounds;
  if (n_buckets == 1) {
    hipError_t e = rlsh::launch_fill_zero_buckets(buckets, n, stream);
    if (e == hipSuccess && n_near_ties != nullptr) e = rlsh::launch_fill_zero_buckets(n_near_ties, 1, stream);
    return hip_status(e, "reformer_lsh_hash");
  }
  const rlsh::HashShape hs = rlsh::make_hash_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets);
  return hip_status(rlsh::launch_hash(qk, dtype == RLSH_BF16, rotations, hs, buckets, n_near_ties, workspace, stream),
                    "reformer_lsh_hash");
}

rlsh_status_t reformer_lsh_hash_noalloc(const void* qk, rlsh_dtype_t dtype, const float* rotations, int batch,
                                        int heads, int seq_len, int d_head, int n_rounds, int n_buckets,
                                        int32_t* buckets, int32_t* n_near_ties, hipStream_t stream) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets, -1);
  if (st != RLSH_OK) return st;
  if ((st = check_dtype(dtype)) != RLSH_OK) return st;
  if (qk == nullptr || buckets == nullptr) return fail(RLSH_ERR_INVALID_ARGUMENT, "qk and buckets must be non-null");
  if ((st = check_aligned(qk, "qk")) != RLSH_OK) return st;
  if (n_buckets == 1) {
    const size_t n = tokens(batch, heads, seq_len) * n_rounds;
    hipError_t e = rlsh::launch_fill_zero_buckets(buckets, n, stream);
    if (e == hipSuccess && n_near_ties != nullptr) e = rlsh::launch_fill_zero_buckets(n_near_ties, 1, stream);
    return hip_status(e, "reformer_lsh_hash_noalloc");
  }
  if (rotations == nullptr) return fail(RLSH_ERR_INVALID_ARGUMENT, "rotations must be non-null when n_buckets > 1");
  const size_t need = hash_ws(batch, heads, seq_len, d_head, n_rounds, n_buckets);
  if (need > static_cast<size_t>(RLSH_NOALLOC_SCRATCH_BYTES))
    return fail(RLSH_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of hash scratch; the static scratch of reformer_lsh_hash_noalloc holds "
                "%zu (use reformer_lsh_hash with a workspace)",
                need, static_cast<size_t>(RLSH_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != RLSH_OK) return st;
  // Nothing in the scratch has to start at zero: the set-up kernel writes the
  // rotation fragments, the transposed copy and the bound maxima, every hash
  // workgroup writes its near-tie count, and the fix-up reads only the entries
  // counted by this call.
  const rlsh::HashShape hs = rlsh::make_hash_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets);
  return hip_status(rlsh::launch_hash(qk, dtype == RLSH_BF16, rotations, hs, buckets, n_near_ties, ws, stream),
                    "reformer_lsh_hash_noalloc");
}

size_t reformer_lsh_sort_workspace_bytes(int batch, int heads, int seq_len, int n_rounds, int n_buckets) {
  if (check_shape(batch, heads, seq_len, -1, n_rounds, n_buckets, -1) != RLSH_OK) return 0;
  return sort_ws(batch, heads, seq_len, n_rounds, n_buckets);
}

rlsh_status_t reformer_lsh_sort(const int32_t* buckets, int batch, int heads, int seq_len, int n_rounds,
                                int n_buckets, int32_t* perm, int32_t* inv_perm, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, -1, n_rounds, n_buckets, -1);
  if (st != RLSH_OK) return st;
  if (buckets == nullptr || perm == nullptr) return fail(RLSH_ERR_INVALID_ARGUMENT, "buckets and perm must be non-null");
  if ((st = check_aligned(workspace, "workspace")) != RLSH_OK) return st;
  const size_t need = sort_ws(batch, heads, seq_len, n_rounds, n_buckets);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(RLSH_ERR_WORKSPACE_TOO_SMALL, "sort workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  const rlsh::SortShape ss = rlsh::make_sort_shape(batch * heads * n_rounds, seq_len, n_buckets);
  return hip_status(rlsh::launch_sort(buckets, ss, perm, inv_perm, workspace, stream), "reformer_lsh_sort");
}

rlsh_status_t reformer_lsh_chunk_attend(const void* qk, const void* v, rlsh_dtype_t dtype, const int32_t* perm,
                                        int batch, int heads, int seq_len, int d_head, int n_rounds, int chunk_len,
                                        int causal, float* o_rounds, float* z_rounds, hipStream_t stream) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, d_head, n_rounds, -1, chunk_len);
  if (st != RLSH_OK) return st;
  if ((st = check_dtype(dtype)) != RLSH_OK) return st;
  if (qk == nullptr || v == nullptr || perm == nullptr || o_rounds == nullptr || z_rounds == nullptr)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "qk, v, perm, o_rounds and z_rounds must be non-null");
  if ((st = check_aligned(qk, "qk")) != RLSH_OK || (st = check_aligned(v, "v")) != RLSH_OK ||
      (st = check_aligned(o_rounds, "o_rounds")) != RLSH_OK)
    return st;
  return hip_status(rlsh::launch_chunk_attend(qk, v, dtype == RLSH_BF16, perm, batch * heads, seq_len, d_head, n_rounds,
                                              chunk_len, causal != 0, o_rounds, z_rounds, stream),
                    "reformer_lsh_chunk_attend");
}

rlsh_status_t reformer_lsh_combine(const float* o_rounds, const float* z_rounds, const void* v, rlsh_dtype_t dtype,
                                   int batch, int heads, int seq_len, int d_head, int n_rounds, void* out,
                                   hipStream_t stream) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, d_head, n_rounds, -1, -1);
  if (st != RLSH_OK) return st;
  if ((st = check_dtype(dtype)) != RLSH_OK) return st;
  if (o_rounds == nullptr || z_rounds == nullptr || v == nullptr || out == nullptr)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "o_rounds, z_rounds, v and out must be non-null");
  if ((st = check_aligned(o_rounds, "o_rounds")) != RLSH_OK || (st = check_aligned(v, "v")) != RLSH_OK ||
      (st = check_aligned(out, "out")) != RLSH_OK)
    return st;
  return hip_status(rlsh::launch_combine(o_rounds, z_rounds, v, dtype == RLSH_BF16, batch * heads, seq_len, d_head,
                                         n_rounds, out, nullptr, stream),
                    "reformer_lsh_combine");
}

size_t reformer_lsh_attend_workspace_bytes(rlsh_dtype_t dtype, int batch, int heads, int seq_len, int d_head,
                                           int n_rounds, int chunk_len) {
  if (check_shape(batch, heads, seq_len, d_head, n_rounds, -1, chunk_len) != RLSH_OK) return 0;
  if (check_dtype(dtype) != RLSH_OK) return 0;
  return attend_ws(dtype, batch, heads, seq_len, d_head, n_rounds, chunk_len);
}

namespace {

rlsh_status_t attend_impl(const void* qk, const void* v, rlsh_dtype_t dtype, const int32_t* perm, int batch,
                          int heads, int seq_len, int d_head, int n_rounds, int chunk_len, int causal, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream, const char* name) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, d_head, n_rounds, -1, chunk_len);
  if (st != RLSH_OK) return st;
  if ((st = check_dtype(dtype)) != RLSH_OK) return st;
  if (qk == nullptr || v == nullptr || perm == nullptr || out == nullptr)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "qk, v, perm and out must be non-null");
  if ((st = check_aligned(qk, "qk")) != RLSH_OK || (st = check_aligned(v, "v")) != RLSH_OK ||
      (st = check_aligned(out, "out")) != RLSH_OK || (st = check_aligned(workspace, "workspace")) != RLSH_OK)
    return st;
  const RoundLayout rl = round_layout(dtype, batch, heads, seq_len, d_head, n_rounds, chunk_len);
  const size_t need = rl.o_bytes + rl.z_bytes;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RLSH_ERR_WORKSPACE_TOO_SMALL, "attend workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  return hip_status(run_attend(qk, v, dtype, perm, batch * heads, seq_len, d_head, n_rounds, chunk_len, causal, out, rl,
                               ws, ws + rl.o_bytes, stream, nullptr, lse),
                    name);
}

}  // namespace

rlsh_status_t reformer_lsh_attend(const void* qk, const void* v, rlsh_dtype_t dtype, const int32_t* perm, int batch,
                                  int heads, int seq_len, int d_head, int n_rounds, int chunk_len, int causal,
                                  void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return attend_impl(qk, v, dtype, perm, batch, heads, seq_len, d_head, n_rounds, chunk_len, causal, out, nullptr,
                     workspace, workspace_bytes, stream, "reformer_lsh_attend");
}

rlsh_status_t reformer_lsh_attend_lse(const void* qk, const void* v, rlsh_dtype_t dtype, const int32_t* perm,
                                      int batch, int heads, int seq_len, int d_head, int n_rounds, int chunk_len,
                                      int causal, void* out, float* lse, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  if (lse == nullptr) return fail(RLSH_ERR_INVALID_ARGUMENT, "lse must be non-null");
  return attend_impl(qk, v, dtype, perm, batch, heads, seq_len, d_head, n_rounds, chunk_len, causal, out, lse,
                     workspace, workspace_bytes, stream, "reformer_lsh_attend_lse");
}

size_t reformer_lsh_workspace_bytes(rlsh_dtype_t dtype, int batch, int heads, int seq_len, int d_head, int n_rounds,
                                    int n_buckets, int chunk_len) {
  if (check_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets, chunk_len) != RLSH_OK) return 0;
  if (check_dtype(dtype) != RLSH_OK) return 0;
  return full_layout(dtype, batch, heads, seq_len, d_head, n_rounds, n_buckets, chunk_len).total;
}

static rlsh_status_t attention_impl(const void* qk, const void* v, const float* rotations, rlsh_dtype_t dtype,
                                    int batch, int heads, int seq_len, int d_head, int n_rounds, int n_buckets,
                                    int chunk_len, int causal, void* out, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream, hipEvent_t* ev) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets, chunk_len);
  if (st != RLSH_OK) return st;
  if ((st = check_dtype(dtype)) != RLSH_OK) return st;
  if (qk == nullptr || v == nullptr || out == nullptr)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "qk, v and out must be non-null");
  if ((st = check_aligned(qk, "qk")) != RLSH_OK || (st = check_aligned(v, "v")) != RLSH_OK ||
      (st = check_aligned(out, "out")) != RLSH_OK || (st = check_aligned(workspace, "workspace")) != RLSH_OK)
    return st;
  if (n_buckets > 1 && rotations == nullptr)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "rotations must be non-null when n_buckets > 1");
  const FullLayout f = full_layout(dtype, batch, heads, seq_len, d_head, n_rounds, n_buckets, chunk_len);
  if (workspace == nullptr || workspace_bytes < f.total)
    return fail(RLSH_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", f.total, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  int32_t* bk = reinterpret_cast<int32_t*>(ws + f.buckets);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + f.perm);
  void* region = ws + f.region;
  const bool bf16 = dtype == RLSH_BF16;
  const int bh = batch * heads;
  hipError_t e = hipSuccess;
  if (ev) e = hipEventRecord(ev[0], stream);
  if (e == hipSuccess && n_buckets > 1) {
    const rlsh::HashShape hs = rlsh::make_hash_shape(batch, heads, seq_len, d_head, n_rounds, n_buckets);
    e = rlsh::launch_hash(qk, bf16, rotations, hs, bk, nullptr, region, stream, ev ? ev + 1 : nullptr);
    if (e == hipSuccess) {
      const rlsh::SortShape ss = rlsh::make_sort_shape(bh * n_rounds, seq_len, n_buckets);
      e = rlsh::launch_sort(bk, ss, perm, nullptr, region, stream);
    }
  } else if (e == hipSuccess) {
    // One bucket: every round keeps the original order.
    for (int i = 1; ev && e == hipSuccess && i <= 3; ++i) e = hipEventRecord(ev[i], stream);
    const rlsh::SortShape ss = rlsh::make_sort_shape(bh * n_rounds, seq_len, 1);
    if (e == hipSuccess) e = rlsh::launch_sort(nullptr, ss, perm, nullptr, nullptr, stream);
  }
  if (e == hipSuccess && ev) e = hipEventRecord(ev[4], stream);
  if (e == hipSuccess)
    e = run_attend(qk, v, dtype, perm, bh, seq_len, d_head, n_rounds, chunk_len, causal, out, f.rounds, region,
                   ws + f.z, stream, ev ? ev + 5 : nullptr);
  if (e == hipSuccess && ev) e = hipEventRecord(ev[6], stream);
  return hip_status(e, "reformer_lsh_attention");
}

rlsh_status_t reformer_lsh_attention(const void* qk, const void* v, const float* rotations, rlsh_dtype_t dtype,
                                     int batch, int heads, int seq_len, int d_head, int n_rounds, int n_buckets,
                                     int chunk_len, int causal, void* out, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  return attention_impl(qk, v, rotations, dtype, batch, heads, seq_len, d_head, n_rounds, n_buckets, chunk_len,
                        causal, out, workspace, workspace_bytes, stream, nullptr);
}

rlsh_status_t reformer_lsh_attention_timed(const void* qk, const void* v, const float* rotations, rlsh_dtype_t dtype,
                                           int batch, int heads, int seq_len, int d_head, int n_rounds, int n_buckets,
                                           int chunk_len, int causal, void* out, void* workspace,
                                           size_t workspace_bytes, hipEvent_t* events, int n_events,
                                           hipStream_t stream) {
  if (events == nullptr || n_events < RLSH_TIMED_EVENTS)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "events must hold %d hipEvent_t", RLSH_TIMED_EVENTS);
  for (int i = 0; i < RLSH_TIMED_EVENTS; ++i)
    if (events[i] == nullptr) return fail(RLSH_ERR_INVALID_ARGUMENT, "events[%d] is null", i);
  return attention_impl(qk, v, rotations, dtype, batch, heads, seq_len, d_head, n_rounds, n_buckets, chunk_len,
                        causal, out, workspace, workspace_bytes, stream, events);
}

rlsh_status_t reformer_lsh_local_attention(const void* q, const void* k, const void* v, rlsh_dtype_t dtype, int batch,
                                           int heads, int seq_len, int d_head, int chunk_len, int n_before,
                                           int n_after, int causal, void* out, hipStream_t stream) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, d_head, 1, -1, chunk_len);
  if (st != RLSH_OK) return st;
  if ((st = check_dtype(dtype)) != RLSH_OK) return st;
  if (n_before < 0 || n_after < 0)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "n_before and n_after must be >= 0 (got %d, %d)", n_before, n_after);
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "q, k, v and out must be non-null");
  if ((st = check_aligned(q, "q")) != RLSH_OK || (st = check_aligned(k, "k")) != RLSH_OK ||
      (st = check_aligned(v, "v")) != RLSH_OK || (st = check_aligned(out, "out")) != RLSH_OK)
    return st;
  // Chunks beyond the sequence do not exist: cap the overlaps (keeps the
  // window arithmetic inside int range for any caller value).
  const int n_chunks = seq_len / std::min(chunk_len, seq_len);
  return hip_status(rlsh::launch_local_attend(q, k, v, dtype == RLSH_BF16, batch * heads, seq_len, d_head, chunk_len,
                                              std::min(n_before, n_chunks), std::min(n_after, n_chunks), causal != 0,
                                              out, stream),
                    "reformer_lsh_local_attention");
}

// Backward needs chunks of exactly 64 slots.
rlsh_status_t check_backward_shape(int seq_len, int chunk_len) {
  if (std::min(chunk_len, seq_len) != 64)
    return fail(RLSH_ERR_UNSUPPORTED, "the backward pass needs chunks of 64 slots (chunk_len %d, seq_len %d)",
                chunk_len, seq_len);
  return ok();
}

size_t reformer_lsh_attend_backward_workspace_bytes(int batch, int heads, int seq_len, int d_head, int n_rounds,
                                                    int chunk_len) {
  if (check_shape(batch, heads, seq_len, d_head, n_rounds, -1, chunk_len) != RLSH_OK) return 0;
  if (check_backward_shape(seq_len, chunk_len) != RLSH_OK) return 0;
  return rlsh::backward_scratch_bytes(batch * heads, seq_len, n_rounds);
}

namespace {

rlsh_status_t backward_impl(const void* qk, const void* v, rlsh_dtype_t dtype, const int32_t* perm, int batch,
                            int heads, int seq_len, int d_head, int n_rounds, int chunk_len, int causal,
                            const void* out, const void* dout, const float* lse, float* dqk, float* dv,
                            void* workspace, size_t workspace_bytes, hipStream_t stream, const char* name) {
  rlsh_status_t st = check_shape(batch, heads, seq_len, d_head, n_rounds, -1, chunk_len);
  if (st != RLSH_OK) return st;
  if ((st = check_dtype(dtype)) != RLSH_OK) return st;
  if ((st = check_backward_shape(seq_len, chunk_len)) != RLSH_OK) return st;
  if (qk == nullptr || v == nullptr || perm == nullptr || out == nullptr || dout == nullptr || dqk == nullptr ||
      dv == nullptr)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "qk, v, perm, out, dout, dqk and dv must be non-null");
  if ((st = check_aligned(qk, "qk")) != RLSH_OK || (st = check_aligned(v, "v")) != RLSH_OK ||
      (st = check_aligned(out, "out")) != RLSH_OK || (st = check_aligned(dout, "dout")) != RLSH_OK ||
      (st = check_aligned(dqk, "dqk")) != RLSH_OK || (st = check_aligned(dv, "dv")) != RLSH_OK ||
      (st = check_aligned(workspace, "workspace")) != RLSH_OK)
    return st;
  const size_t need = rlsh::backward_scratch_bytes(batch * heads, seq_len, n_rounds);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RLSH_ERR_WORKSPACE_TOO_SMALL, "backward workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  return hip_status(rlsh::launch_attend_backward(qk, v, dtype == RLSH_BF16, perm, batch * heads, seq_len, d_head,
                                                 n_rounds, causal != 0, out, dout, lse, dqk, dv, workspace, stream),
                    name);
}

}  // namespace

rlsh_status_t reformer_lsh_attend_backward(const void* qk, const void* v, rlsh_dtype_t dtype, const int32_t* perm,
                                           int batch, int heads, int seq_len, int d_head, int n_rounds,
                                           int chunk_len, int causal, const void* out, const void* dout, float* dqk,
                                           float* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return backward_impl(qk, v, dtype, perm, batch, heads, seq_len, d_head, n_rounds, chunk_len, causal, out, dout,
                       nullptr, dqk, dv, workspace, workspace_bytes, stream, "reformer_lsh_attend_backward");
}

rlsh_status_t reformer_lsh_attend_backward_lse(const void* qk, const void* v, rlsh_dtype_t dtype,
                                               const int32_t* perm, int batch, int heads, int seq_len, int d_head,
                                               int n_rounds, int chunk_len, int causal, const void* out,
                                               const void* dout, const float* lse, float* dqk, float* dv,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (lse == nullptr) return fail(RLSH_ERR_INVALID_ARGUMENT, "lse must be non-null");
  return backward_impl(qk, v, dtype, perm, batch, heads, seq_len, d_head, n_rounds, chunk_len, causal, out, dout, lse,
                       dqk, dv, workspace, workspace_bytes, stream, "reformer_lsh_attend_backward_lse");
}

rlsh_status_t check_ff_shape(int n_tokens, int d_model, int d_ff, int chunk_tokens) {
  if (n_tokens < 1 || chunk_tokens < 0)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "n_tokens must be >= 1 and chunk_tokens >= 0 (got %d, %d)", n_tokens,
                chunk_tokens);
  if (d_model < 128 || d_ff < 128 || d_model % 128 != 0 || d_ff % 128 != 0)
    return fail(RLSH_ERR_UNSUPPORTED, "d_model and d_ff must be positive multiples of 128 (got %d, %d)", d_model, d_ff);
  return ok();
}

size_t reformer_lsh_feed_forward_workspace_bytes(int n_tokens, int d_model, int d_ff, int chunk_tokens) {
  if (check_ff_shape(n_tokens, d_model, d_ff, chunk_tokens) != RLSH_OK) return 0;
  return a256(rlsh::feed_forward_chunk(n_tokens, chunk_tokens) * d_ff * sizeof(uint16_t));
}

rlsh_status_t reformer_lsh_feed_forward(const void* x, const void* w1, const float* b1, const void* w2,
                                        const float* b2, int n_tokens, int d_model, int d_ff, int chunk_tokens,
                                        void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rlsh_status_t st = check_ff_shape(n_tokens, d_model, d_ff, chunk_tokens);
  if (st != RLSH_OK) return st;
  if (x == nullptr || w1 == nullptr || b1 == nullptr || w2 == nullptr || b2 == nullptr || out == nullptr)
    return fail(RLSH_ERR_INVALID_ARGUMENT, "x, w1, b1, w2, b2 and out must be non-null");
  if ((st = check_aligned(x, "x")) != RLSH_OK || (st = check_aligned(w1, "w1")) != RLSH_OK ||
      (st = check_aligned(b1, "b1")) != RLSH_OK || (st = check_aligned(w2, "w2")) != RLSH_OK ||
      (st = check_aligned(b2, "b2")) != RLSH_OK || (st = check_aligned(out, "out")) != RLSH_OK ||
      (st = check_aligned(workspace, "workspace")) != RLSH_OK)
    return st;
  const size_t need = reformer_lsh_feed_forward_workspace_bytes(n_tokens, d_model, d_ff, chunk_tokens);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RLSH_ERR_WORKSPACE_TOO_SMALL, "feed-forward workspace needs %zu bytes (got %zu)", need,
                workspace_bytes);
  return hip_status(rlsh::launch_feed_forward(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w1), b1,
                                              static_cast<const uint16_t*>(w2), b2, n_tokens, d_model, d_ff,
                                              chunk_tokens, static_cast<uint16_t*>(out),
                                              static_cast<uint16_t*>(workspace), stream),
                    "reformer_lsh_feed_forward");
}

}  // extern "C"
