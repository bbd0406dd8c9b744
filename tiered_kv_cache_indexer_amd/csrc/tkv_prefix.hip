// Cold-prefix records and rehydration into the mirror (FreeToken PR #525,
// "What the patch does", items 2-4): a prefix leaving the tier is copied out
// (its logical ids get reused); on a later hit it comes back host to host
// into the offloader's mirror, and the LRU's fetch on selection covers
// residency.  A record is a page's mirror row followed by its indexer slab
// entries for every layer: bf16 values [L][Hkv*d] and the fp64 key sums
// [L][Hkv*d] (the running sum a partly written page's later tokens add to).
//
// The rows move host to host (threads over memcpy); only the slab entries,
// 10 bytes per feature, cross the host link, in slices of 128 pages.
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "tkv_dev.h"
#include "tkv_launch.h"

namespace {

__global__ __launch_bounds__(TKV_BLOCK) void k_slab_gather(DevCtx c, const int32_t* pages, uint16_t* vals,
                                                           double* sums) {
  const int i = blockIdx.x, l = blockIdx.y, n_layers = gridDim.y;
  const int E = c.Hkv * c.D;
  const size_t src = ((size_t)l * c.N + pages[i]) * E, dst = ((size_t)i * n_layers + l) * E;
  for (int e = threadIdx.x; e < E; e += TKV_BLOCK) {
    vals[dst + e] = c.slab[src + e];
    sums[dst + e] = c.slab_acc[src + e];
  }
}

__global__ __launch_bounds__(TKV_BLOCK) void k_slab_scatter(DevCtx c, const int32_t* pages, const uint16_t* vals,
                                                            const double* sums) {
  const int i = blockIdx.x, l = blockIdx.y, n_layers = gridDim.y;
  const int E = c.Hkv * c.D;
  const size_t dst = ((size_t)l * c.N + pages[i]) * E, src = ((size_t)i * n_layers + l) * E;
  for (int e = threadIdx.x; e < E; e += TKV_BLOCK) {
    c.slab[dst + e] = vals[src + e];
    c.slab_acc[dst + e] = sums[src + e];
  }
}

// A restored id that is resident loses its slot (the slot holds the id's
// previous content); the slot keeps its stamp, so it is reused in LRU order.
__global__ void k_unbind(DevCtx c, const int32_t* pages, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int p = pages[i];
  const int s = c.page_to_slot[p];
  if (s >= 0) {
    c.page_to_slot[p] = -1;
    c.slot_to_page[s] = -1;
  }
}

}  // namespace

// Copies rows between the mirror and records with up to `max_threads` host
// threads (1: in the calling thread, no thread objects created).
void prefix_copy_rows(uint8_t* dst, size_t dst_stride, const uint8_t* src, size_t src_stride, size_t row_bytes,
                      const int32_t* pages, int n, bool to_mirror, int max_threads) {
  const int T = std::max(1, std::min(max_threads, n / 4));
  auto work = [&](int t) {
    for (int i = t; i < n; i += T) {
      const size_t p = (size_t)pages[i];
      if (to_mirror) std::memcpy(dst + p * dst_stride, src + (size_t)i * src_stride, row_bytes);
      else std::memcpy(dst + (size_t)i * dst_stride, src + p * src_stride, row_bytes);
    }
  };
  if (T == 1) {
    work(0);
    return;
  }
  std::vector<std::thread> th;
  for (int t = 0; t < T; ++t) th.emplace_back(work, t);
  for (auto& x : th) x.join();
}

hipError_t launch_slab_gather(const DevCtx& c, const int32_t* pages, int n, uint16_t* vals, double* sums,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_slab_gather, dim3(n, c.L), dim3(TKV_BLOCK), 0, st, c, pages, vals, sums);
  return hipGetLastError();
}

hipError_t launch_slab_scatter(const DevCtx& c, const int32_t* pages, int n, const uint16_t* vals,
                               const double* sums, hipStream_t st) {
  hipLaunchKernelGGL(k_slab_scatter, dim3(n, c.L), dim3(TKV_BLOCK), 0, st, c, pages, vals, sums);
  return hipGetLastError();
}

hipError_t launch_unbind(const DevCtx& c, const int32_t* pages, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_unbind, dim3((n + 255) / 256), dim3(256), 0, st, c, pages, n);
  return hipGetLastError();
}
