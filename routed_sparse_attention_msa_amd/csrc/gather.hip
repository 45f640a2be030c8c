// S4: gather of the selected documents' pooled K/V.
//
// Method: MSA README (EverMind-AI/MSA), "Inference Pipeline" stage 2 -- only
// the selected documents' pooled K/V are loaded and placed next to the local
// context; the content tier may live in host DRAM and be fetched on demand.
//
// A workgroup copies a slice of one selected document's C pooled rows of K
// and V (contiguous in the bank) with 16-byte loads and stores: 4 KiB from
// device memory, the whole document from pinned host memory.  The source may be
// device memory or pinned host memory mapped into the GPU's address space
// (then the loads travel over the host link with no host round trip).  Ids
// outside [0, n_docs) are never dereferenced: their rows are zero-filled and
// an optional error word is raised (the dormouse ADR-0014 page records a
// gather that faulted on out-of-range indices; this kernel cannot).
#include "internal.h"

namespace msa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gather_kernel(
    const char* __restrict__ kbar, const char* __restrict__ vbar, const int32_t* __restrict__ ids,
    int k, int64_t n_docs, size_t doc_bytes, size_t slice_bytes, int slices, char* __restrict__ k_sel,
    char* __restrict__ v_sel,
    int* __restrict__ err_flag) {
  // one workgroup per (selected document, slice of `slice_bytes` of its rows)
  const int b = blockIdx.y, i = blockIdx.x / slices, sl = blockIdx.x % slices;
  const int64_t id = ids[(size_t)b * k + i];
  const size_t dst = ((size_t)b * k + i) * doc_bytes;
  const bool ok = id >= 0 && id < n_docs;
  if (!ok && err_flag != nullptr && threadIdx.x == 0) atomicOr(err_flag, 1);
  const size_t src = ok ? (size_t)id * doc_bytes : 0;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const size_t end = min(doc_bytes, (size_t)(sl + 1) * slice_bytes);
  for (size_t off = (size_t)sl * slice_bytes + threadIdx.x * 16; off < end; off += (size_t)kThreads * 16) {
    const u32x4 kv = ok ? load16(kbar + src + off) : zero;
    const u32x4 vv = ok ? load16(vbar + src + off) : zero;
    store16(k_sel + dst + off, kv);
    store16(v_sel + dst + off, vv);
  }
}

}  // namespace

hipError_t launch_gather(const void* kbar, const void* vbar, const int32_t* ids, int batch, int k,
                         int64_t n_docs, int cpd, size_t row_bytes, bool host_src, void* k_sel, void* v_sel,
                         int* err_flag, hipStream_t s) {
  const size_t doc_bytes = (size_t)cpd * row_bytes;
  // Device memory: one 4 KiB slice per workgroup, so every load of the copy
  // is in flight at once (16 documents of 16 KiB: 4.4 -> 2.6 us).  Pinned
  // host memory: one workgroup streams a whole document (the host link served
  // the scattered 4 KiB slices slower: 64 documents, 53.6 against 43.1 us).
  const size_t slice_bytes = host_src ? doc_bytes : (size_t)kThreads * 16;
  const size_t slices = (doc_bytes + slice_bytes - 1) / slice_bytes;
  if ((size_t)k * slices > 0x7FFFFFFFu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(k * slices), batch), dim3(kThreads), 0, s,
                     static_cast<const char*>(kbar), static_cast<const char*>(vbar), ids, k, n_docs,
                     doc_bytes, slice_bytes, (int)slices, static_cast<char*>(k_sel), static_cast<char*>(v_sel),
                     err_flag);
  return hipGetLastError();
}

}  // namespace msa
