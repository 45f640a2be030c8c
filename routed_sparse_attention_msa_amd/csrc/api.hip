// The extern "C" boundary of libmsa: argument validation, workspace sizing,
// error reporting, and the host-tier fetch engine.  Every compute step runs
// in the HIP kernels behind the launch_* functions.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_last_error = "no error";

msa_status fail(msa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

msa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSA_OK;
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_size(msa_dtype dt) { return dt == MSA_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == MSA_F32 || dt == MSA_BF16; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

#define CHECK_ARG(cond, ...)                                   \
  do {                                                         \
    if (!(cond)) return fail(MSA_ERR_INVALID, __VA_ARGS__);    \
  } while (0)

// Library-owned, per-device resources of the host tier and of the checked
// gather.  Each device has one side stream and a pool of staging slots; a
// call takes a slot for its own use (events, a pinned id buffer, an error
// word), so concurrent calls never share one.  The pool lock is held only to
// take or return a slot, never across a wait.  Objects are created on first
// use, owned through unique_ptr (their addresses never move) and kept until
// the process ends.
struct Slot {
  hipEvent_t ready = nullptr;    // recorded on the caller's stream when the call starts
  hipEvent_t on_host = nullptr;  // the ids (or the error word) have reached the host
  hipEvent_t done = nullptr;     // the slot's host-tier copies have finished
  int32_t* host_ids = nullptr;   // pinned
  size_t host_ids_cap = 0;
  int* dev_flag = nullptr;       // device error word of a checked gather
  int* host_flag = nullptr;      // pinned copy of it
};

struct DeviceRes {
  hipStream_t side = nullptr;
  std::vector<std::unique_ptr<Slot>> free_slots;
};

std::mutex g_res_mutex;
std::map<int, std::unique_ptr<DeviceRes>> g_res;

msa_status new_slot(std::unique_ptr<Slot>* out) {
  auto slot = std::make_unique<Slot>();
  hipError_t e;
  for (hipEvent_t* ev : {&slot->ready, &slot->on_host, &slot->done})
    if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return hip_status(e, "hipEventCreate");
  if ((e = hipMalloc(&slot->dev_flag, sizeof(int))) != hipSuccess) return hip_status(e, "hipMalloc(flag)");
  if ((e = hipHostMalloc(&slot->host_flag, sizeof(int), hipHostMallocDefault)) != hipSuccess)
    return hip_status(e, "hipHostMalloc(flag)");
  *out = std::move(slot);
  return MSA_OK;
}

// A slot of the current device, returned to its pool when the guard ends.
class SlotGuard {
 public:
  msa_status acquire() {
    hipError_t e = hipGetDevice(&dev_);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    {
      std::lock_guard<std::mutex> lock(g_res_mutex);
      std::unique_ptr<DeviceRes>& r = g_res[dev_];
      if (!r) r = std::make_unique<DeviceRes>();
      if (r->side == nullptr &&
          (e = hipStreamCreateWithFlags(&r->side, hipStreamNonBlocking)) != hipSuccess)
        return hip_status(e, "hipStreamCreate");
      side_ = r->side;
      if (!r->free_slots.empty()) {
        slot_ = std::move(r->free_slots.back());
        r->free_slots.pop_back();
        return MSA_OK;
      }
    }
    return new_slot(&slot_);  // created outside the lock
  }
  ~SlotGuard() {
    if (!slot_) return;
    std::lock_guard<std::mutex> lock(g_res_mutex);
    g_res[dev_]->free_slots.push_back(std::move(slot_));
  }
  Slot* slot() { return slot_.get(); }
  hipStream_t side() const { return side_; }

 private:
  int dev_ = 0;
  hipStream_t side_ = nullptr;
  std::unique_ptr<Slot> slot_;
};

// Device-visible address of pinned host memory, or an error for pageable memory.
msa_status host_device_ptr(const void* p, const void** dptr) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MSA_ERR_INVALID, "host-tier source %p is not pinned host memory", p);
  }
  if (attr.type != hipMemoryTypeHost)
    return fail(MSA_ERR_INVALID, "host-tier source %p is not pinned host memory (type %d)", p,
                (int)attr.type);
  *dptr = attr.devicePointer != nullptr ? attr.devicePointer : p;
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_abi_version(void) { return 1; }

const char* msa_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
msa_status msa_pool_chunks(const void* x, void* xbar, float* xbar_norm, int64_t n_docs,
                           int32_t doc_len, int32_t chunk, int32_t heads, int32_t dim,
                           msa_dtype dt, void* stream) {
  CHECK_ARG(valid_dtype(dt), "unknown dtype %d", (int)dt);
  CHECK_ARG(n_docs >= 0 && doc_len > 0 && chunk > 0 && heads > 0 && dim > 0,
            "sizes must be positive (n_docs=%lld doc_len=%d chunk=%d heads=%d dim=%d)",
            (long long)n_docs, doc_len, chunk, heads, dim);
  CHECK_ARG(doc_len % chunk == 0, "doc_len %d is not a multiple of chunk %d", doc_len, chunk);
  const size_t es = dtype_size(dt);
  CHECK_ARG(((size_t)heads * dim * es) % 16 == 0, "heads*dim*sizeof(dtype) must be a multiple of 16");
  if (xbar_norm != nullptr) {
    const int64_t hb = (int64_t)dim * (int64_t)es;
    CHECK_ARG(is_pow2(hb) && hb >= 16 && hb <= 1024,
              "with norms, dim*sizeof(dtype) must be a power of two in [16, 1024] (got %lld)",
              (long long)hb);
    CHECK_ARG(aligned16(xbar_norm) || ((uintptr_t)xbar_norm & 3u) == 0, "xbar_norm misaligned");
  }
  if (n_docs == 0) return MSA_OK;
  CHECK_ARG(x && xbar, "null tensor pointer");
  CHECK_ARG(aligned16(x) && aligned16(xbar), "x and xbar must be 16-byte aligned");
  const int64_t n_chunks = n_docs * (doc_len / chunk);
  CHECK_ARG(n_chunks < (int64_t)1 << 31, "too many chunks");
  return hip_status(msa::launch_pool(x, xbar, xbar_norm, n_chunks, chunk, heads, dim, dt,
                                     static_cast<hipStream_t>(stream)),
                    "msa_pool_chunks launch");
}

// ---------------------------------------------------------------------------
msa_status msa_chunk_offsets(const int64_t* doc_off, int64_t n_docs, int32_t chunk,
                             int64_t* chunk_off, void* stream) {
  CHECK_ARG(n_docs >= 0 && chunk > 0, "n_docs must be >= 0 and chunk > 0 (n_docs=%lld chunk=%d)",
            (long long)n_docs, chunk);
  CHECK_ARG(doc_off && chunk_off, "null pointer");
  CHECK_ARG(((uintptr_t)doc_off & 7u) == 0 && ((uintptr_t)chunk_off & 7u) == 0, "offsets misaligned");
  return hip_status(msa::launch_chunk_offsets(doc_off, n_docs, chunk, chunk_off,
                                              static_cast<hipStream_t>(stream)),
                    "msa_chunk_offsets launch");
}

msa_status msa_encode_docs(const void* x, void* xbar, float* xbar_norm, const int64_t* doc_off,
                           const int64_t* chunk_off, int64_t n_docs, int64_t total_rows,
                           int64_t total_chunks, int32_t chunk, int32_t heads, int32_t dim,
                           float rope_base, msa_dtype dt, void* stream) {
  CHECK_ARG(valid_dtype(dt), "unknown dtype %d", (int)dt);
  CHECK_ARG(n_docs >= 0 && total_rows >= 0 && total_chunks >= 0 && chunk > 0 && heads > 0 && dim > 0,
            "sizes must be positive (n_docs=%lld total_rows=%lld total_chunks=%lld chunk=%d heads=%d dim=%d)",
            (long long)n_docs, (long long)total_rows, (long long)total_chunks, chunk, heads, dim);
  CHECK_ARG(rope_base >= 0.f && rope_base == rope_base, "rope_base must be >= 0 (0: no rotation)");
  const size_t es = dtype_size(dt);
  CHECK_ARG(((size_t)heads * dim * es) % 16 == 0, "heads*dim*sizeof(dtype) must be a multiple of 16");
  if (xbar_norm != nullptr || rope_base > 0.f) {
    const int64_t hb = (int64_t)dim * (int64_t)es;
    CHECK_ARG(is_pow2(hb) && hb >= 32 && hb <= 1024,
              "with norms or RoPE, dim*sizeof(dtype) must be a power of two in [32, 1024] (got %lld)",
              (long long)hb);
  }
  CHECK_ARG(xbar_norm == nullptr || ((uintptr_t)xbar_norm & 3u) == 0, "xbar_norm misaligned");
  if (n_docs == 0 || total_chunks == 0) return MSA_OK;
  CHECK_ARG(x && xbar && doc_off && chunk_off, "null pointer");
  CHECK_ARG(aligned16(x) && aligned16(xbar), "x and xbar must be 16-byte aligned");
  CHECK_ARG(((uintptr_t)doc_off & 7u) == 0 && ((uintptr_t)chunk_off & 7u) == 0, "offsets misaligned");
  return hip_status(msa::launch_encode(x, xbar, xbar_norm, doc_off, chunk_off, n_docs, total_rows,
                                       total_chunks, chunk, heads, dim, rope_base, dt,
                                       static_cast<hipStream_t>(stream)),
                    "msa_encode_docs launch");
}

// ---------------------------------------------------------------------------
static msa_status check_route(int32_t batch, int32_t q_len, int32_t heads, int32_t dim,
                              int64_t n_docs, int32_t cpd, msa_dtype dt) {
  CHECK_ARG(valid_dtype(dt), "unknown dtype %d", (int)dt);
  CHECK_ARG(batch > 0 && q_len > 0 && heads > 0 && dim > 0 && n_docs > 0 && cpd > 0,
            "sizes must be positive");
  CHECK_ARG(n_docs < (int64_t)1 << 31 && n_docs * cpd < (int64_t)1 << 31, "bank too large");
  CHECK_ARG(((size_t)dim * dtype_size(dt)) % 16 == 0, "dim*sizeof(dtype) must be a multiple of 16");
  return MSA_OK;
}

msa_status msa_route_scores_workspace(int32_t batch, int32_t q_len, int32_t heads, int32_t dim,
                                      int64_t n_docs, int32_t chunks_per_doc, msa_dtype dt,
                                      size_t* bytes) {
  msa_status st = check_route(batch, q_len, heads, dim, n_docs, chunks_per_doc, dt);
  if (st != MSA_OK) return st;
  CHECK_ARG(bytes != nullptr, "bytes is null");
  *bytes = msa::route_workspace_bytes(batch, q_len, heads, dim, n_docs, chunks_per_doc, dt);
  return MSA_OK;
}

msa_status msa_route_scores(const void* q_r, const void* kbar_r, const float* kbar_r_norm,
                            int32_t batch, int32_t q_len, int32_t heads, int32_t dim,
                            int64_t n_docs, int32_t chunks_per_doc, msa_dtype dt,
                            float* doc_scores, void* ws, size_t ws_bytes, void* stream) {
  msa_status st = check_route(batch, q_len, heads, dim, n_docs, chunks_per_doc, dt);
  if (st != MSA_OK) return st;
  CHECK_ARG(q_r && kbar_r && kbar_r_norm && doc_scores, "null tensor pointer");
  CHECK_ARG(aligned16(q_r) && aligned16(kbar_r) && aligned16(kbar_r_norm) && aligned16(doc_scores),
            "tensors must be 16-byte aligned");
  const size_t need = msa::route_workspace_bytes(batch, q_len, heads, dim, n_docs, chunks_per_doc, dt);
  CHECK_ARG(ws_bytes >= need, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  CHECK_ARG(need == 0 || (ws != nullptr && aligned16(ws)), "workspace pointer missing or misaligned");
  return hip_status(msa::launch_route(q_r, kbar_r, kbar_r_norm, batch, q_len, heads, dim, n_docs,
                                      chunks_per_doc, dt, doc_scores, ws,
                                      static_cast<hipStream_t>(stream)),
                    "msa_route_scores launch");
}

msa_status msa_route_scores_noalloc(const void* q_r, const void* kbar_r, const float* kbar_r_norm,
                                    int32_t batch, int32_t q_len, int32_t heads, int32_t dim, int64_t n_docs,
                                    int32_t chunks_per_doc, msa_dtype dt, float* doc_scores, void* stream) {
  msa_status st = check_route(batch, q_len, heads, dim, n_docs, chunks_per_doc, dt);
  if (st != MSA_OK) return st;
  CHECK_ARG(q_r && kbar_r && kbar_r_norm && doc_scores, "null tensor pointer");
  CHECK_ARG(aligned16(q_r) && aligned16(kbar_r) && aligned16(kbar_r_norm) && aligned16(doc_scores),
            "tensors must be 16-byte aligned");
  const size_t need = msa::route_workspace_bytes(batch, q_len, heads, dim, n_docs, chunks_per_doc, dt);
  CHECK_ARG(need <= msa::kRouteStaticScratchBytes,
            "this call needs %zu bytes of scratch, above the %zu bytes the library holds per device; use "
            "msa_route_scores with a workspace", need, msa::kRouteStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = msa::route_static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "routing scratch lookup");
  }
  return hip_status(msa::launch_route(q_r, kbar_r, kbar_r_norm, batch, q_len, heads, dim, n_docs,
                                      chunks_per_doc, dt, doc_scores, ws, static_cast<hipStream_t>(stream)),
                    "msa_route_scores_noalloc launch");
}

// ---------------------------------------------------------------------------
static msa_status check_topk(int32_t batch, int64_t n_docs, int32_t k) {
  CHECK_ARG(batch > 0 && n_docs > 0, "sizes must be positive");
  CHECK_ARG(n_docs < (int64_t)1 << 31, "n_docs must be below 2^31");
  CHECK_ARG(k >= 1 && k <= n_docs && k <= 1024, "k=%d must lie in [1, min(n_docs, 1024)]", k);
  return MSA_OK;
}

msa_status msa_topk_docs_workspace(int32_t batch, int64_t n_docs, int32_t k, size_t* bytes) {
  msa_status st = check_topk(batch, n_docs, k);
  if (st != MSA_OK) return st;
  CHECK_ARG(bytes != nullptr, "bytes is null");
  *bytes = msa::topk_workspace_bytes(batch, n_docs, k);
  return MSA_OK;
}

msa_status msa_topk_docs(const float* doc_scores, int32_t batch, int64_t n_docs, int32_t k,
                         int32_t* topk_ids, float* topk_scores, void* ws, size_t ws_bytes,
                         void* stream) {
  msa_status st = check_topk(batch, n_docs, k);
  if (st != MSA_OK) return st;
  CHECK_ARG(doc_scores && topk_ids, "null tensor pointer");
  const size_t need = msa::topk_workspace_bytes(batch, n_docs, k);
  CHECK_ARG(ws_bytes >= need, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  CHECK_ARG(need == 0 || (ws != nullptr && aligned16(ws)), "workspace pointer missing or misaligned");
  return hip_status(msa::launch_topk(doc_scores, batch, n_docs, k, topk_ids, topk_scores, ws,
                                     static_cast<hipStream_t>(stream)),
                    "msa_topk_docs launch");
}

// ---------------------------------------------------------------------------
// Multi-round routing (Memory Interleave)

// Exclusion entries may share the output buffer only in the multi-round
// layout: equal row strides, each row's k outputs after its own n_excl
// exclusion entries and before the next row.
static bool excl_layout_ok(const int32_t* excl, int64_t es, int n_excl, const int32_t* out, int64_t os,
                           int k, int batch) {
  if (excl == nullptr || n_excl == 0) return true;
  const int32_t* e_end = excl + (size_t)(batch - 1) * (size_t)es + n_excl;
  const int32_t* o_end = out + (size_t)(batch - 1) * (size_t)os + k;
  if (e_end <= out || o_end <= excl) return true;
  if (es != os) return false;
  const ptrdiff_t d = out - excl;
  return d >= n_excl && d + k <= es;
}

msa_status msa_topk_docs_excluding(const float* doc_scores, int32_t batch, int64_t n_docs, int32_t k,
                                   const int32_t* excl_ids, int32_t n_excl, int64_t excl_stride,
                                   int32_t* topk_ids, float* topk_scores, int64_t out_stride, void* ws,
                                   size_t ws_bytes, void* stream) {
  msa_status st = check_topk(batch, n_docs, k);
  if (st != MSA_OK) return st;
  CHECK_ARG(n_excl >= 0 && (int64_t)k + n_excl <= n_docs,
            "need n_excl >= 0 and k + n_excl <= n_docs (k=%d n_excl=%d n_docs=%lld)", k, n_excl,
            (long long)n_docs);
  CHECK_ARG(n_excl == 0 || (excl_ids != nullptr && excl_stride >= n_excl),
            "excl_ids missing or excl_stride < n_excl");
  CHECK_ARG(out_stride >= k, "out_stride < k");
  CHECK_ARG(doc_scores && topk_ids, "null tensor pointer");
  CHECK_ARG(((uintptr_t)topk_ids & 3u) == 0 && ((uintptr_t)excl_ids & 3u) == 0, "id arrays misaligned");
  CHECK_ARG(excl_layout_ok(excl_ids, excl_stride, n_excl, topk_ids, out_stride, k, batch),
            "exclusion entries overlap the outputs");
  const size_t need = msa::topk_workspace_bytes(batch, n_docs, k);
  CHECK_ARG(ws_bytes >= need, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  CHECK_ARG(need == 0 || (ws != nullptr && aligned16(ws)), "workspace pointer missing or misaligned");
  return hip_status(msa::launch_topk_excl(doc_scores, batch, n_docs, k, excl_ids, n_excl, excl_stride,
                                          topk_ids, topk_scores, out_stride, ws,
                                          static_cast<hipStream_t>(stream)),
                    "msa_topk_docs_excluding launch");
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Every round's router queries are given up front and a round's scores do not
// depend on the earlier rounds' picks, so all rounds can be routed in one
// launch over rounds*batch sequences -- done when the tiled kernel routes both
// that launch and a single round (its scores of a sequence are then the same
// bits as a round's own call; the other paths may order a sum differently for
// another number of sequences).
static bool rounds_fused(int32_t rounds, int32_t batch, int32_t q_len, int32_t heads, int32_t dim, int32_t cpd,
                         msa_dtype dt) {
  return rounds > 1 && (int64_t)rounds * batch <= 65535 && msa::route_is_tiled(batch, q_len, heads, dim, cpd, dt) &&
         msa::route_is_tiled(rounds * batch, q_len, heads, dim, cpd, dt);
}

static msa_status rounds_workspace(int32_t rounds, int32_t batch, int32_t q_len, int32_t heads,
                                   int32_t dim, int64_t n_docs, int32_t cpd, int32_t k, msa_dtype dt,
                                   size_t* scores_bytes, size_t* total) {
  msa_status st = check_route(batch, q_len, heads, dim, n_docs, cpd, dt);
  if (st != MSA_OK) return st;
  if ((st = check_topk(batch, n_docs, k)) != MSA_OK) return st;
  CHECK_ARG(rounds >= 1 && (int64_t)rounds * k <= n_docs,
            "need rounds >= 1 and rounds*k <= n_docs (rounds=%d k=%d n_docs=%lld)", rounds, k,
            (long long)n_docs);
  *scores_bytes = align256((size_t)rounds * batch * (size_t)n_docs * sizeof(float));
  const size_t route_ws = rounds_fused(rounds, batch, q_len, heads, dim, cpd, dt)
                              ? msa::route_workspace_bytes(rounds * batch, q_len, heads, dim, n_docs, cpd, dt)
                              : msa::route_workspace_bytes(batch, q_len, heads, dim, n_docs, cpd, dt);
  *total = *scores_bytes + std::max(route_ws, msa::topk_workspace_bytes(batch, n_docs, k));
  return MSA_OK;
}

msa_status msa_route_rounds_workspace(int32_t rounds, int32_t batch, int32_t q_len, int32_t heads,
                                      int32_t dim, int64_t n_docs, int32_t chunks_per_doc, int32_t k,
                                      msa_dtype dt, size_t* bytes) {
  size_t sb = 0, total = 0;
  msa_status st = rounds_workspace(rounds, batch, q_len, heads, dim, n_docs, chunks_per_doc, k, dt, &sb,
                                   &total);
  if (st != MSA_OK) return st;
  CHECK_ARG(bytes != nullptr, "bytes is null");
  *bytes = total;
  return MSA_OK;
}

msa_status msa_route_rounds(const void* q_r, const void* kbar_r, const float* kbar_r_norm,
                            int32_t rounds, int32_t batch, int32_t q_len, int32_t heads, int32_t dim,
                            int64_t n_docs, int32_t chunks_per_doc, int32_t k, msa_dtype dt,
                            int32_t* topk_ids, float* topk_scores, void* ws, size_t ws_bytes,
                            void* stream) {
  size_t sb = 0, total = 0;
  msa_status st = rounds_workspace(rounds, batch, q_len, heads, dim, n_docs, chunks_per_doc, k, dt, &sb,
                                   &total);
  if (st != MSA_OK) return st;
  CHECK_ARG(q_r && kbar_r && kbar_r_norm && topk_ids, "null tensor pointer");
  CHECK_ARG(aligned16(q_r) && aligned16(kbar_r) && aligned16(kbar_r_norm), "tensors must be 16-byte aligned");
  CHECK_ARG(((uintptr_t)topk_ids & 3u) == 0 && ((uintptr_t)topk_scores & 3u) == 0, "outputs misaligned");
  CHECK_ARG(ws_bytes >= total, "workspace too small (%zu < %zu bytes)", ws_bytes, total);
  CHECK_ARG(ws != nullptr && aligned16(ws), "workspace pointer missing or misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* scores = static_cast<float*>(ws);      // [rounds][batch][n_docs]
  void* scratch = static_cast<char*>(ws) + sb;
  const int64_t stride = (int64_t)rounds * k;
  const size_t q_bytes = (size_t)batch * q_len * heads * dim * dtype_size(dt);
  const bool fused = rounds_fused(rounds, batch, q_len, heads, dim, chunks_per_doc, dt);
  hipError_t e = hipSuccess;
  if (fused) {   // all rounds' scores in one routing launch: q_r is [rounds * batch] sequences
    e = msa::launch_route(q_r, kbar_r, kbar_r_norm, rounds * batch, q_len, heads, dim, n_docs, chunks_per_doc,
                          dt, scores, scratch, s);
    if (e != hipSuccess) return hip_status(e, "msa_route_rounds route launch");
  }
  for (int r = 0; r < rounds; ++r) {
    float* sc = scores + (size_t)r * batch * n_docs;
    if (!fused) {
      e = msa::launch_route(static_cast<const char*>(q_r) + (size_t)r * q_bytes, kbar_r, kbar_r_norm, batch, q_len,
                            heads, dim, n_docs, chunks_per_doc, dt, sc, scratch, s);
      if (e != hipSuccess) return hip_status(e, "msa_route_rounds route launch");
    }
    e = msa::launch_topk_excl(sc, batch, n_docs, k, topk_ids, r * k, stride, topk_ids + (size_t)r * k,
                              topk_scores ? topk_scores + (size_t)r * k : nullptr, stride, scratch, s);
    if (e != hipSuccess) return hip_status(e, "msa_route_rounds top-k launch");
  }
  return MSA_OK;
}

// ---------------------------------------------------------------------------
msa_status msa_gather_kv(const void* kbar, const void* vbar, int32_t src_on_host,
                         const int32_t* topk_ids, int32_t batch, int32_t k, int64_t n_docs,
                         int32_t chunks_per_doc, int32_t heads_kv, int32_t dim, msa_dtype dt,
                         void* k_sel, void* v_sel, int32_t flags, void* stream) {
  CHECK_ARG(valid_dtype(dt), "unknown dtype %d", (int)dt);
  CHECK_ARG(batch > 0 && k > 0 && n_docs > 0 && chunks_per_doc > 0 && heads_kv > 0 && dim > 0,
            "sizes must be positive");
  CHECK_ARG((flags & ~(MSA_GATHER_CHECKED | MSA_GATHER_HOST_MEMCPY)) == 0, "unknown flags 0x%x", flags);
  CHECK_ARG(kbar && vbar && topk_ids && k_sel && v_sel, "null tensor pointer");
  const size_t row_bytes = (size_t)heads_kv * dim * dtype_size(dt);
  CHECK_ARG(row_bytes % 16 == 0, "heads_kv*dim*sizeof(dtype) must be a multiple of 16");
  CHECK_ARG(aligned16(kbar) && aligned16(vbar) && aligned16(k_sel) && aligned16(v_sel),
            "tensors must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t doc_bytes = (size_t)chunks_per_doc * row_bytes;
  hipError_t e;

  if (src_on_host && (flags & MSA_GATHER_HOST_MEMCPY)) {
    // Per-document copies on the side stream; the host must know the ids first.
    const void* dk;
    const void* dv;
    msa_status st = host_device_ptr(kbar, &dk);
    if (st != MSA_OK) return st;
    if ((st = host_device_ptr(vbar, &dv)) != MSA_OK) return st;
    SlotGuard guard;
    if ((st = guard.acquire()) != MSA_OK) return st;
    Slot* sl = guard.slot();
    hipStream_t side = guard.side();
    const size_t n_ids = (size_t)batch * k;
    if (sl->host_ids_cap < n_ids) {
      if (sl->host_ids) (void)hipHostFree(sl->host_ids);
      sl->host_ids = nullptr;
      sl->host_ids_cap = 0;
      if ((e = hipHostMalloc(&sl->host_ids, n_ids * sizeof(int32_t), hipHostMallocDefault)) != hipSuccess)
        return hip_status(e, "hipHostMalloc(ids)");
      sl->host_ids_cap = n_ids;
    }
    // The ids are final once the work already queued on `s` has run: mark that
    // point with an event and bring the ids back on the side stream, so the
    // host waits for exactly that work (not for anything queued on `s` later,
    // nor for other threads' calls).
    if ((e = hipEventRecord(sl->ready, s)) != hipSuccess) return hip_status(e, "event record");
    if ((e = hipStreamWaitEvent(side, sl->ready, 0)) != hipSuccess) return hip_status(e, "side wait");
    if ((e = hipMemcpyAsync(sl->host_ids, topk_ids, n_ids * sizeof(int32_t), hipMemcpyDeviceToHost, side)) !=
        hipSuccess)
      return hip_status(e, "ids D2H");
    if ((e = hipEventRecord(sl->on_host, side)) != hipSuccess) return hip_status(e, "event record");
    if ((e = hipEventSynchronize(sl->on_host)) != hipSuccess) return hip_status(e, "ids wait");
    for (size_t i = 0; i < n_ids; ++i) {
      const int64_t id = sl->host_ids[i];
      if (id < 0 || id >= n_docs)
        return fail(MSA_ERR_INVALID, "document id %lld at position %zu out of range [0, %lld)",
                    (long long)id, i, (long long)n_docs);
    }
    const char* hk = static_cast<const char*>(kbar);
    const char* hv = static_cast<const char*>(vbar);
    for (size_t i = 0; i < n_ids; ++i) {
      const size_t src = (size_t)sl->host_ids[i] * doc_bytes;
      const size_t dst = i * doc_bytes;
      if ((e = hipMemcpyAsync(static_cast<char*>(k_sel) + dst, hk + src, doc_bytes, hipMemcpyHostToDevice,
                              side)) != hipSuccess)
        return hip_status(e, "K fetch");
      if ((e = hipMemcpyAsync(static_cast<char*>(v_sel) + dst, hv + src, doc_bytes, hipMemcpyHostToDevice,
                              side)) != hipSuccess)
        return hip_status(e, "V fetch");
    }
    if ((e = hipEventRecord(sl->done, side)) != hipSuccess) return hip_status(e, "event record");
    if ((e = hipStreamWaitEvent(s, sl->done, 0)) != hipSuccess) return hip_status(e, "stream wait");
    return MSA_OK;
  }

  const void* src_k = kbar;
  const void* src_v = vbar;
  if (src_on_host) {
    msa_status st = host_device_ptr(kbar, &src_k);
    if (st != MSA_OK) return st;
    if ((st = host_device_ptr(vbar, &src_v)) != MSA_OK) return st;
  }
  if (!(flags & MSA_GATHER_CHECKED)) {
    e = msa::launch_gather(src_k, src_v, topk_ids, batch, k, n_docs, chunks_per_doc, row_bytes, src_on_host,
                           k_sel, v_sel, nullptr, s);
    return hip_status(e, "msa_gather_kv launch");
  }
  // Checked: this call's own error word, cleared, raised by the kernel, read back.
  SlotGuard guard;
  msa_status st = guard.acquire();
  if (st != MSA_OK) return st;
  Slot* sl = guard.slot();
  if ((e = hipMemsetAsync(sl->dev_flag, 0, sizeof(int), s)) != hipSuccess) return hip_status(e, "flag clear");
  e = msa::launch_gather(src_k, src_v, topk_ids, batch, k, n_docs, chunks_per_doc, row_bytes, src_on_host, k_sel,
                         v_sel, sl->dev_flag, s);
  if (e != hipSuccess) return hip_status(e, "msa_gather_kv launch");
  if ((e = hipMemcpyAsync(sl->host_flag, sl->dev_flag, sizeof(int), hipMemcpyDeviceToHost, s)) != hipSuccess)
    return hip_status(e, "flag read");
  if ((e = hipEventRecord(sl->on_host, s)) != hipSuccess) return hip_status(e, "event record");
  if ((e = hipEventSynchronize(sl->on_host)) != hipSuccess) return hip_status(e, "flag wait");
  if (*sl->host_flag != 0) return fail(MSA_ERR_INVALID, "a document id was outside [0, %lld)", (long long)n_docs);
  return MSA_OK;
}

// ---------------------------------------------------------------------------
static msa_status check_attn(int32_t batch, int32_t q_len, int32_t heads_q, int32_t heads_kv,
                             int32_t dim, int32_t mem_len, int32_t loc_len, msa_dtype dt) {
  CHECK_ARG(valid_dtype(dt), "unknown dtype %d", (int)dt);
  CHECK_ARG(batch > 0 && q_len > 0 && heads_q > 0 && heads_kv > 0 && dim > 0 && mem_len >= 0,
            "sizes must be positive");
  CHECK_ARG(heads_q % heads_kv == 0, "heads_q %d is not a multiple of heads_kv %d", heads_q, heads_kv);
  CHECK_ARG(loc_len >= q_len, "loc_len %d must be >= q_len %d", loc_len, q_len);
  CHECK_ARG(dim <= 256, "dim %d above 256 is not supported", dim);
  CHECK_ARG(((size_t)dim * dtype_size(dt)) % 16 == 0, "dim*sizeof(dtype) must be a multiple of 16");
  // The kernels address one sequence's memory, local and query rows through
  // 32-bit buffer offsets: each span must stay below 4 GiB.
  const int64_t kv_row = (int64_t)heads_kv * dim * (int64_t)dtype_size(dt);
  const int64_t q_row = (int64_t)heads_q * dim * (int64_t)dtype_size(dt);
  CHECK_ARG((int64_t)mem_len * kv_row < ((int64_t)1 << 32) && (int64_t)loc_len * kv_row < ((int64_t)1 << 32) &&
                (int64_t)q_len * q_row < ((int64_t)1 << 32),
            "one sequence's memory, local or query rows span 4 GiB or more");
  return MSA_OK;
}

msa_status msa_sparse_attn_workspace(int32_t batch, int32_t q_len, int32_t heads_q,
                                     int32_t heads_kv, int32_t dim, int32_t mem_len,
                                     int32_t loc_len, msa_dtype dt, size_t* bytes) {
  msa_status st = check_attn(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dt);
  if (st != MSA_OK) return st;
  CHECK_ARG(bytes != nullptr, "bytes is null");
  *bytes = msa::attn_workspace_bytes(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dt);
  return MSA_OK;
}

msa_status msa_sparse_attn(const void* q, const void* k_sel, const void* v_sel, int32_t mem_len,
                           const void* k_loc, const void* v_loc, int32_t loc_len, int32_t batch,
                           int32_t q_len, int32_t heads_q, int32_t heads_kv, int32_t dim,
                           float scale, msa_dtype dt, void* out, float* lse, void* ws,
                           size_t ws_bytes, void* stream) {
  msa_status st = check_attn(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dt);
  if (st != MSA_OK) return st;
  CHECK_ARG(q && k_loc && v_loc && out, "null tensor pointer");
  CHECK_ARG(mem_len == 0 || (k_sel && v_sel), "k_sel/v_sel required when mem_len > 0");
  CHECK_ARG(aligned16(q) && aligned16(k_loc) && aligned16(v_loc) && aligned16(out) &&
                (mem_len == 0 || (aligned16(k_sel) && aligned16(v_sel))),
            "tensors must be 16-byte aligned");
  CHECK_ARG(scale == scale && scale > 0.f, "scale must be positive");
  const size_t need = msa::attn_workspace_bytes(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dt);
  CHECK_ARG(ws_bytes >= need, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  CHECK_ARG(need == 0 || (ws != nullptr && aligned16(ws)), "workspace pointer missing or misaligned");
  return hip_status(msa::launch_attn(q, k_sel, v_sel, mem_len, k_loc, v_loc, loc_len, batch, q_len,
                                     heads_q, heads_kv, dim, scale, dt, out, lse, ws,
                                     static_cast<hipStream_t>(stream)),
                    "msa_sparse_attn launch");
}

msa_status msa_attn_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b,
                          int32_t batch, int32_t q_len, int32_t heads_q, int32_t dim, msa_dtype dt, void* out,
                          float* lse, void* stream) {
  CHECK_ARG(valid_dtype(dt), "unknown dtype %d", (int)dt);
  CHECK_ARG(batch > 0 && q_len > 0 && heads_q > 0 && dim > 0, "sizes must be positive");
  CHECK_ARG(dim <= 256, "dim %d above 256 is not supported", dim);
  CHECK_ARG(((size_t)dim * dtype_size(dt)) % 16 == 0, "dim*sizeof(dtype) must be a multiple of 16");
  CHECK_ARG(out_a && lse_a && out_b && lse_b && out, "null tensor pointer");
  CHECK_ARG(aligned16(out_a) && aligned16(out_b) && aligned16(out), "out_a, out_b and out must be 16-byte aligned");
  CHECK_ARG(((uintptr_t)lse_a & 3u) == 0 && ((uintptr_t)lse_b & 3u) == 0 && ((uintptr_t)lse & 3u) == 0,
            "lse arrays must be 4-byte aligned");
  return hip_status(msa::launch_attn_merge(out_a, lse_a, out_b, lse_b, batch, q_len, heads_q, dim, dt, out, lse,
                                           static_cast<hipStream_t>(stream)),
                    "msa_attn_merge launch");
}

msa_status msa_sparse_attn_backward_workspace(int32_t batch, int32_t q_len, int32_t heads_q,
                                              int32_t heads_kv, int32_t dim, int32_t mem_len,
                                              int32_t loc_len, msa_dtype dt, size_t* bytes) {
  msa_status st = check_attn(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dt);
  if (st != MSA_OK) return st;
  CHECK_ARG(bytes != nullptr, "bytes is null");
  *bytes = msa::attn_backward_workspace_bytes(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dt);
  return MSA_OK;
}

msa_status msa_sparse_attn_backward(const void* q, const void* k_sel, const void* v_sel, int32_t mem_len,
                                    const void* k_loc, const void* v_loc, int32_t loc_len, const void* out,
                                    const void* d_out, const float* lse, int32_t batch, int32_t q_len,
                                    int32_t heads_q, int32_t heads_kv, int32_t dim, float scale,
                                    msa_dtype dt, void* d_q, void* d_k_sel, void* d_v_sel, void* d_k_loc,
                                    void* d_v_loc, void* ws, size_t ws_bytes, void* stream) {
  msa_status st = check_attn(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dt);
  if (st != MSA_OK) return st;
  CHECK_ARG(q && k_loc && v_loc && out && d_out && lse && d_q && d_k_loc && d_v_loc, "null tensor pointer");
  CHECK_ARG(mem_len == 0 || (k_sel && v_sel && d_k_sel && d_v_sel),
            "k_sel/v_sel and their gradients required when mem_len > 0");
  CHECK_ARG(aligned16(q) && aligned16(k_loc) && aligned16(v_loc) && aligned16(out) && aligned16(d_out) &&
                aligned16(lse) && aligned16(d_q) && aligned16(d_k_loc) && aligned16(d_v_loc) &&
                (mem_len == 0 || (aligned16(k_sel) && aligned16(v_sel) && aligned16(d_k_sel) &&
                                  aligned16(d_v_sel))),
            "tensors must be 16-byte aligned");
  CHECK_ARG(scale == scale && scale > 0.f, "scale must be positive");
  const size_t need = msa::attn_backward_workspace_bytes(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dt);
  CHECK_ARG(ws_bytes >= need, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  CHECK_ARG(ws != nullptr && aligned16(ws), "workspace pointer missing or misaligned");
  return hip_status(msa::launch_attn_backward(q, k_sel, v_sel, mem_len, k_loc, v_loc, loc_len, out, d_out,
                                              lse, batch, q_len, heads_q, heads_kv, dim, scale, dt, d_q,
                                              d_k_sel, d_v_sel, d_k_loc, d_v_loc, ws,
                                              static_cast<hipStream_t>(stream)),
                    "msa_sparse_attn_backward launch");
}

// ---------------------------------------------------------------------------
// Workspace sizing by operation: dims are the per-operation call's integer
// arguments in order (the dtype as its msa_dtype value).
static bool fits_i32(int64_t v) { return v >= INT32_MIN && v <= INT32_MAX; }

msa_status msa_workspace_size(int32_t op, const int64_t* dims, int32_t ndims, size_t* bytes) {
  CHECK_ARG(bytes != nullptr, "bytes is null");
  CHECK_ARG(ndims >= 0 && (ndims == 0 || dims != nullptr), "dims missing");
  auto need = [&](int n) { return ndims == n; };
  auto i32 = [&](int i) { return (int32_t)dims[i]; };
  for (int i = 0; i < ndims; ++i) {
    // n_docs (an int64_t argument) may exceed int32; it is range-checked by the op
    const bool wide = (op == MSA_OP_ROUTE_SCORES && i == 4) || (op == MSA_OP_TOPK_DOCS && i == 1) ||
                      (op == MSA_OP_TOPK_DOCS_EXCLUDING && i == 1) || (op == MSA_OP_ROUTE_ROUNDS && i == 5);
    CHECK_ARG(wide || fits_i32(dims[i]), "dims[%d] = %lld is out of the int32 range", i, (long long)dims[i]);
  }
  switch (op) {
    case MSA_OP_POOL_CHUNKS:
    case MSA_OP_ENCODE_DOCS:
    case MSA_OP_GATHER_KV:
    case MSA_OP_GDN_STATE_SUM:
    case MSA_OP_GATED_DELTA_RULE:
    case MSA_OP_GATED_DELTA_RULE_CHUNKED:
      *bytes = 0;  // these operations use no scratch
      return MSA_OK;
    case MSA_OP_ROUTE_SCORES:
      CHECK_ARG(need(7), "MSA_OP_ROUTE_SCORES takes 7 dims (got %d)", ndims);
      return msa_route_scores_workspace(i32(0), i32(1), i32(2), i32(3), dims[4], i32(5), (msa_dtype)i32(6),
                                        bytes);
    case MSA_OP_TOPK_DOCS:
    case MSA_OP_TOPK_DOCS_EXCLUDING:
      CHECK_ARG(need(3), "MSA_OP_TOPK_DOCS takes 3 dims (got %d)", ndims);
      return msa_topk_docs_workspace(i32(0), dims[1], i32(2), bytes);
    case MSA_OP_ROUTE_ROUNDS:
      CHECK_ARG(need(9), "MSA_OP_ROUTE_ROUNDS takes 9 dims (got %d)", ndims);
      return msa_route_rounds_workspace(i32(0), i32(1), i32(2), i32(3), i32(4), dims[5], i32(6), i32(7),
                                        (msa_dtype)i32(8), bytes);
    case MSA_OP_SPARSE_ATTN:
      CHECK_ARG(need(8), "MSA_OP_SPARSE_ATTN takes 8 dims (got %d)", ndims);
      return msa_sparse_attn_workspace(i32(0), i32(1), i32(2), i32(3), i32(4), i32(5), i32(6), (msa_dtype)i32(7),
                                       bytes);
    case MSA_OP_SPARSE_ATTN_BACKWARD:
      CHECK_ARG(need(8), "MSA_OP_SPARSE_ATTN_BACKWARD takes 8 dims (got %d)", ndims);
      return msa_sparse_attn_backward_workspace(i32(0), i32(1), i32(2), i32(3), i32(4), i32(5), i32(6),
                                                (msa_dtype)i32(7), bytes);
    default:
      return fail(MSA_ERR_INVALID, "unknown operation %d", op);
  }
}

// ---------------------------------------------------------------------------
// Linear-layer variant
msa_status msa_gdn_state_sum(const float* doc_states, const int32_t* topk_ids, int32_t batch, int32_t k,
                             int64_t n_docs, int32_t heads, int32_t dk, int32_t dv, float* s_ext, void* stream) {
  CHECK_ARG(batch > 0 && k > 0 && n_docs > 0 && heads > 0 && dk > 0 && dv > 0, "sizes must be positive");
  CHECK_ARG(batch <= 65535, "batch above 65535 is not supported");
  CHECK_ARG(((int64_t)heads * dk * dv) % 4 == 0, "heads*dk*dv must be a multiple of 4");
  CHECK_ARG(doc_states && topk_ids && s_ext, "null tensor pointer");
  CHECK_ARG(aligned16(doc_states) && aligned16(s_ext) && ((uintptr_t)topk_ids & 3u) == 0,
            "tensors must be 16-byte aligned");
  return hip_status(msa::launch_gdn_state_sum(doc_states, topk_ids, batch, k, n_docs, (int64_t)heads * dk * dv,
                                              s_ext, static_cast<hipStream_t>(stream)),
                    "msa_gdn_state_sum launch");
}

msa_status msa_gated_delta_rule(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                float scale, const float* initial_state, int32_t batch, int32_t seq_len,
                                int32_t heads, int32_t dk, int32_t dv, msa_dtype dt, void* out,
                                float* final_state, void* stream) {
  CHECK_ARG(valid_dtype(dt), "unknown dtype %d", (int)dt);
  CHECK_ARG(batch > 0 && seq_len >= 0 && heads > 0 && dv > 0, "sizes must be positive");
  CHECK_ARG(dk == 64 || dk == 128, "dk must be 64 or 128 (got %d)", dk);
  CHECK_ARG(batch <= 65535 && heads <= 65535, "batch and heads must be at most 65535");
  CHECK_ARG(out != nullptr || final_state != nullptr, "nothing to compute: out and final_state are both NULL");
  CHECK_ARG(scale == scale, "scale is NaN");
  CHECK_ARG(seq_len == 0 || (k && v && g && beta && (out == nullptr || q)), "null tensor pointer");
  if (seq_len == 0 && final_state == nullptr) return MSA_OK;
  return hip_status(msa::launch_gdn(q, k, v, g, beta, scale, initial_state, batch, seq_len, heads, dk, dv, dt, out,
                                    final_state, static_cast<hipStream_t>(stream)),
                    "msa_gated_delta_rule launch");
}

msa_status msa_gated_delta_rule_chunked(const void* q, const void* k, const void* v, const float* g,
                                        const float* beta, float scale, const float* initial_state, int32_t batch,
                                        int32_t seq_len, int32_t heads, int32_t dk, int32_t dv, msa_dtype dt,
                                        void* out, float* final_state, void* stream) {
  CHECK_ARG(dt == MSA_BF16, "the chunked form takes bf16 q / k / v (got dtype %d)", (int)dt);
  CHECK_ARG(dk == 128 && dv == 128, "the chunked form takes dk = dv = 128 (got %d, %d)", dk, dv);
  CHECK_ARG(batch > 0 && seq_len >= 0 && heads > 0, "sizes must be positive");
  CHECK_ARG(batch <= 65535, "batch above 65535 is not supported");
  CHECK_ARG((int64_t)seq_len * heads * 128 * 2 < ((int64_t)1 << 32),
            "a sequence's rows (seq_len * heads * 256 bytes) must span less than 4 GiB");
  CHECK_ARG(out != nullptr || final_state != nullptr, "nothing to compute: out and final_state are both NULL");
  CHECK_ARG(scale == scale, "scale is NaN");
  CHECK_ARG(seq_len == 0 || (k && v && g && beta && (out == nullptr || q)), "null tensor pointer");
  CHECK_ARG(aligned16(k) && (out == nullptr || aligned16(q)), "q and k must be 16-byte aligned");
  CHECK_ARG(((uintptr_t)v & 1u) == 0 && ((uintptr_t)out & 1u) == 0 && ((uintptr_t)g & 3u) == 0 &&
                ((uintptr_t)beta & 3u) == 0 && ((uintptr_t)initial_state & 3u) == 0 &&
                ((uintptr_t)final_state & 3u) == 0,
            "tensors must be aligned to their element size");
  if (seq_len == 0 && final_state == nullptr) return MSA_OK;
  return hip_status(msa::launch_gdn_chunked(q, k, v, g, beta, scale, initial_state, batch, seq_len, heads, out,
                                            final_state, static_cast<hipStream_t>(stream)),
                    "msa_gated_delta_rule_chunked launch");
}

}  // extern "C"
