// Fused host->device page copy, write-ensure sampling, state initialisation
// and the codec test kernels (gfx950).
//
// FreeToken PR #499, "Design": one launch copies K+V of a page for every
// layer; PR #525 commit summary: the copy also carries the scale banks.  With
// page-major rows (a row holds one page for all layers, scales included) one
// miss is one contiguous mirror row -> one contiguous pool slot.
//
// The miss count lives on the device, so the launch is fixed-shape: a grid of
// FETCH_GRID workgroups walks (miss, 64 KiB chunk) work items up to
// *miss_count; inside an item each thread moves one 16-byte vector per
// iteration (non-temporal load from the pinned mirror, store to the slot).
// Measured on MI355X over PCIe Gen5 x16: one vector in flight per thread with
// 64 KiB items reads host memory at ~56 GB/s (the contiguous hipMemcpy rate),
// four vectors per thread with 16 KiB items at ~49 GB/s.  Grid sweep on a
// chunk of 4,096 tokens fetching 65,536 cached ones into an empty pool (the
// first layer's fetch, 812 MB): 128 workgroups 14.19 ms, 256 14.15 ms,
// 512 14.18 ms, 1,024 14.61 ms; on a 196k-context decode step from an empty
// pool 256 and 512 tie and 128 is 2.7% slower.
#include <utility>

#include "tkv_dev.h"
#include "tkv_launch.h"

#ifndef FETCH_GRID
#define FETCH_GRID 256
#endif
#ifndef FETCH_CHUNK
#define FETCH_CHUNK (64 * 1024)
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(TKV_BLOCK) void k_fetch(DevCtx c, const int32_t* miss,
                                                     const int32_t* miss_count, int width) {
  int m = *miss_count;
  if (m > width) m = width;
  const int64_t row = c.row_bytes;
  const int cpr = (int)((row + FETCH_CHUNK - 1) / FETCH_CHUNK);
  const int64_t items = (int64_t)m * cpr;
  if (blockIdx.x == 0 && threadIdx.x == 0 && m > 0)
    c.hdr->counters[CNT_BYTES_FETCHED] += (int64_t)m * row;
  const int64_t nvec = row / 16;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int mi = (int)(it / cpr), ch = (int)(it - (int64_t)mi * cpr);
    const int slot = miss[2 * mi], page = miss[2 * mi + 1];
    if (slot < 0 || slot >= c.S || page < 0 || (int64_t)page >= c.N) {
      if (threadIdx.x == 0) set_error(c.hdr, DERR_BAD_MISS);
      continue;
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(c.mirror + (size_t)page * row);
    u32x4* dst = reinterpret_cast<u32x4*>(c.pool + (size_t)slot * row);
    const int64_t v_end = min(nvec, (int64_t)(ch + 1) * (FETCH_CHUNK / 16));
    for (int64_t v = (int64_t)ch * (FETCH_CHUNK / 16) + threadIdx.x; v < v_end; v += TKV_BLOCK)
      dst[v] = __builtin_nontemporal_load(src + v);
  }
}

hipError_t launch_fetch(const DevCtx& c, const int32_t* miss, const int32_t* miss_count, int width,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_fetch, dim3(FETCH_GRID), dim3(TKV_BLOCK), 0, st, c, miss, miss_count, width);
  return hipGetLastError();
}

// ------------------------------------------------------- split row copy ----
// The same copy in parts, for decode steps whose link time should hide the
// compute around it: one part moves, for every miss, one or two layers'
// slices of the row (the layer being decoded, whose attention reads it, and
// the next one); the other moves the rest of the rows, skipping those
// slices.  The parts together move the bytes of k_fetch and leave the same
// pool rows.

// Slices `s0` and `s1` of every missed row (equal: one slice): a flat
// grid-stride walk over the 16-byte vectors of all of them on SLICE_GRID
// workgroups.  With `keep` set, block 0 also stores the miss count and list
// there ([0] = count, then the pairs) for the part that follows.  The grid
// is an eighth of k_fetch's: this copy shares the link with the previous
// call's rest copy, and with 1,024 workgroups (every vector of a few dozen
// misses in flight at once) the two together moved 52.3 GB/s on MI355X; with
// 64-384 workgroups 53.7-54.4 GB/s (+3.5% decode steps at 196k context, with
// 16 or 12 rest workgroups alike); more loads per thread gained nothing.
// Decode steps by grid (batch-4 / 196k thrash, ms): 64 1.354 / 5.08, 96-128
// 1.36 / 5.066, 192 1.38 / 5.07, 256 1.39 / 5.08, 512 1.39 / 5.13, 1,024
// 1.39 / 5.23.
#ifndef SLICE_GRID
#define SLICE_GRID 128
#endif
__global__ __launch_bounds__(TKV_BLOCK) void k_fetch_slice(DevCtx c, const int32_t* miss, const int32_t* miss_count,
                                                           int width, int s0, int s1, int32_t* keep) {
  int m = *miss_count;
  if (m > width) m = width;
  if (keep && blockIdx.x == 0) {
    for (int i = threadIdx.x; i < 2 * m; i += TKV_BLOCK) keep[1 + i] = miss[i];
    if (threadIdx.x == 0) keep[0] = m;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && m > 0) c.hdr->counters[CNT_BYTES_FETCHED] += (int64_t)m * c.row_bytes;
  // 32-bit indices: max_width < 2^16 and two layer slices are at most 2^15 vectors
  const uint32_t nvl = (uint32_t)(c.layer_bytes / 16);
  const uint32_t per = (s0 == s1 ? 1u : 2u) * nvl;
  const uint32_t total = (uint32_t)m * per;
  for (uint32_t v = blockIdx.x * TKV_BLOCK + threadIdx.x; v < total; v += gridDim.x * TKV_BLOCK) {
    const int mi = (int)(v / per);
    const uint32_t e = v - (uint32_t)mi * per;
    const int64_t r = e < nvl ? (int64_t)s0 * nvl + e : (int64_t)s1 * nvl + (e - nvl);
    const int slot = miss[2 * mi], page = miss[2 * mi + 1];
    if (slot < 0 || slot >= c.S || page < 0 || (int64_t)page >= c.N) {
      set_error(c.hdr, DERR_BAD_MISS);
      continue;
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(c.mirror + (size_t)page * c.row_bytes);
    u32x4* dst = reinterpret_cast<u32x4*>(c.pool + (size_t)slot * c.row_bytes);
    dst[r] = __builtin_nontemporal_load(src + r);
  }
}

// Every slice of the kept rows but slices `sa` <= `sb` (equal: one skipped),
// on a small grid: the copy runs beside the decode's kernels, and
// a grid spread over every CU holds enough host reads in flight to stall
// their memory accesses (measured: attention 10 -> 200+ us), while 16
// workgroups still keep the link busy.  Timed call by call on MI355X: 8-16
// workgroups with 4-12 loads per thread move 51-53 GB/s, 32 workgroups 48,
// 48-64 workgroups 43: more host reads in flight slow the link down.
//
// The stall is per XCD: a host read in flight holds a place in the queue of
// its XCD's L2 towards the fabric, and other loads of that XCD that miss
// wait behind it.  Measured with a probe: a 48-workgroup 3 MB HBM read takes
// 1.3 us alone, 23 us beside this copy spread over the XCDs (8 loads per
// thread), 6 us with 2 loads per thread at the same 56 GB/s, and 4.0 against
// 4.1 us when the copy runs on one XCD and the read on the others.  Putting
// the copy on one XCD and the decode's kernels on the other seven (work
// claimed by the workgroups placed there) lost in the decode steps: the
// confined copy moved about half as many bytes beside the decode's kernels,
// and the claims cost the selection more than it gained.
#ifndef REST_GRID
#define REST_GRID 16
#endif
// Calls with at least REST_MIN_ITEMS 64 KiB items per workgroup: each wave
// claims (miss, 16 KiB) pieces from a counter (the next claim in flight while
// it copies) with REST_UNROLL loads in flight per thread, so the waves finish
// together (static (miss, 64 KiB) items per workgroup left the last items to
// a few workgroups: the 196k thrash 5.06-5.10 -> 4.99 ms per step with 16
// loads, 5.00-5.01 with 8).  Smaller calls: (miss, 16 KiB) items dealt to
// the workgroups in turn, REST_SMALL_UNROLL loads in flight.
#ifndef REST_UNROLL
#define REST_UNROLL 16
#endif
#ifndef REST_CHUNK
#define REST_CHUNK FETCH_CHUNK
#endif
#ifndef REST_MIN_ITEMS
#define REST_MIN_ITEMS 12
#endif
// loads in flight per thread with the small items: fewer host reads in
// flight stall the decode's kernels less (measured on the batch-4 workload,
// where the copy is not the critical path: 2 loads 1.43-1.44 ms per step, 4
// or 8 loads 1.48-1.53) and the link stays as busy
#ifndef REST_SMALL_UNROLL
#define REST_SMALL_UNROLL 2
#endif


// Vectors [v_begin, v_end) of the rest of one row, U loads in flight per
// thread: rest vector x is row vector x, stepped over slice sa, then sb.
template <int U>
__device__ __forceinline__ void rest_copy_vectors(const u32x4* src, u32x4* dst, int64_t v_begin, int64_t v_end,
                                                  int64_t a, int64_t b, int64_t nvl, bool two) {
  for (int64_t v0 = v_begin + threadIdx.x; v0 < v_end; v0 += TKV_BLOCK * U) {
    u32x4 t[U];
    int64_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t x = v0 + u * TKV_BLOCK;
      if (x >= a) x += nvl;
      if (two && x >= b) x += nvl;
      r[u] = x;
      if (v0 + u * TKV_BLOCK < v_end) t[u] = __builtin_nontemporal_load(src + x);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * TKV_BLOCK < v_end) dst[r[u]] = t[u];
  }
}

// As rest_copy_vectors, for one wave over its own piece.
template <int U>
__device__ __forceinline__ void wave_copy_vectors(const u32x4* src, u32x4* dst, int64_t v_begin, int64_t v_end,
                                                  int64_t a, int64_t b, int64_t nvl, bool two, int lane) {
  for (int64_t v0 = v_begin + lane; v0 < v_end; v0 += 64 * U) {
    u32x4 t[U];
    int64_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t x = v0 + u * 64;
      if (x >= a) x += nvl;
      if (two && x >= b) x += nvl;
      r[u] = x;
      if (v0 + u * 64 < v_end) t[u] = __builtin_nontemporal_load(src + x);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * 64 < v_end) dst[r[u]] = t[u];
  }
}

__global__ __launch_bounds__(TKV_BLOCK) void k_fetch_rest(DevCtx c, const int32_t* keep, int width, int sa, int sb) {
  int m = keep[0];
  if (m > width) m = width;
  const int32_t* miss = keep + 1;
  const int64_t nvl = c.layer_bytes / 16;
  const int64_t a = (int64_t)sa * nvl, b = (int64_t)sb * nvl;
  const int64_t nvec = c.row_bytes / 16 - (sa == sb ? 1 : 2) * nvl;
  // the call's volume in REST_CHUNK items decides the path
  const int64_t big = (int64_t)m * ((nvec + REST_CHUNK / 16 - 1) / (REST_CHUNK / 16));
  const bool large = big >= (int64_t)REST_MIN_ITEMS * gridDim.x;
  if (large) {
    // pieces claimed by waves; the last wave to finish resets the counters
    constexpr int PV = 1024;                                 // vectors per piece
    const int ppr = (int)((nvec + PV - 1) / PV);
    const int64_t pieces = (int64_t)m * ppr;
    const int lane = threadIdx.x & 63;
    int32_t* q = c.rest_ctr;
    int it = 0;
    if (lane == 0) it = __hip_atomic_fetch_add(&q[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    it = __builtin_amdgcn_readfirstlane(it);
    while (it < pieces) {
      int nxt = 0;
      if (lane == 0) nxt = __hip_atomic_fetch_add(&q[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int mi = (int)(it / ppr), ch = it - mi * ppr;
      const int slot = miss[2 * mi], page = miss[2 * mi + 1];
      if (slot < 0 || slot >= c.S || page < 0 || (int64_t)page >= c.N) {
        if (lane == 0) set_error(c.hdr, DERR_BAD_MISS);
      } else {
        const u32x4* src = reinterpret_cast<const u32x4*>(c.mirror + (size_t)page * c.row_bytes);
        u32x4* dst = reinterpret_cast<u32x4*>(c.pool + (size_t)slot * c.row_bytes);
        const int64_t v_end = min(nvec, (int64_t)(ch + 1) * PV);
        wave_copy_vectors<REST_UNROLL>(src, dst, (int64_t)ch * PV, v_end, a, b, nvl, sb != sa, lane);
      }
      it = __builtin_amdgcn_readfirstlane(nxt);
    }
    if (lane == 0) {
      const int waves = (int)gridDim.x * (TKV_BLOCK / 64);
      if (__hip_atomic_fetch_add(&q[1], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == waves - 1) {
        __hip_atomic_store(&q[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&q[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }
  const int64_t cvec = REST_CHUNK / 64;
  const int cpr = (int)((nvec + cvec - 1) / cvec);
  const int64_t items = (int64_t)m * cpr;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int mi = (int)(it / cpr), ch = (int)(it - (int64_t)mi * cpr);
    const int slot = miss[2 * mi], page = miss[2 * mi + 1];
    if (slot < 0 || slot >= c.S || page < 0 || (int64_t)page >= c.N) {
      if (threadIdx.x == 0) set_error(c.hdr, DERR_BAD_MISS);
      continue;
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(c.mirror + (size_t)page * c.row_bytes);
    u32x4* dst = reinterpret_cast<u32x4*>(c.pool + (size_t)slot * c.row_bytes);
    const int64_t v_begin = (int64_t)ch * cvec, v_end = min(nvec, v_begin + cvec);
    rest_copy_vectors<REST_SMALL_UNROLL>(src, dst, v_begin, v_end, a, b, nvl, sb != sa);
  }
}

hipError_t launch_fetch_slice(const DevCtx& c, const int32_t* miss, const int32_t* miss_count, int width, int s0,
                              int s1, int32_t* keep, hipStream_t st) {
  hipLaunchKernelGGL(k_fetch_slice, dim3(SLICE_GRID), dim3(TKV_BLOCK), 0, st, c, miss, miss_count, width, s0, s1,
                     keep);
  return hipGetLastError();
}

hipError_t launch_fetch_rest(const DevCtx& c, const int32_t* keep, int width, int sa, int sb, hipStream_t st) {
  if (sa > sb) std::swap(sa, sb);
  hipLaunchKernelGGL(k_fetch_rest, dim3(REST_GRID), dim3(TKV_BLOCK), 0, st, c, keep, width, sa, sb);
  return hipGetLastError();
}

// ---------------------------------------------------------- write-ensure ----
// Stride samples start, start+PS, ... plus one boundary sample start+len-1
// per run: every page the run touches is sampled at least once, in page order.
__global__ void k_write_samples(DevCtx c, int n_runs, const int32_t* run_req, const int32_t* run_start,
                                const int32_t* run_len, int spr, const int32_t* bt, int max_pages,
                                const int32_t* old_len) {
  const int W = n_runs * spr;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < W; j += gridDim.x * blockDim.x) {
    const int r = j / spr, k = j - r * spr;
    const int req = run_req[r], start = run_start[r], len = run_len[r];
    int pos = -1;
    if (len > 0) {
      if (k < spr - 1) {
        if (k * c.PS < len) pos = start + k * c.PS;
      } else {
        pos = start + len - 1;
        // the stride samples reach pages start/PS .. start/PS + spr-2 only
        if ((start + len - 1) / c.PS - start / c.PS >= spr) set_error(c.hdr, DERR_RUN_LEN);
      }
    }
    int needed = -1;
    uint8_t nf = 0;
    if (pos >= 0) {
      const int lp = pos / c.PS;
      if (lp < max_pages) {
        needed = bt[(size_t)req * max_pages + lp];
        nf = (lp * c.PS >= old_len[req]) ? 1 : 0;
      } else {
        needed = -2;  // flagged by the ensure as out of range
      }
    }
    c.wneeded[j] = needed;
    c.wnofetch[j] = nf;
  }
}

hipError_t launch_write_ensure(const DevCtx& c, int n_runs, const int32_t* run_req,
                               const int32_t* run_start, const int32_t* run_len, int spr,
                               const int32_t* bt, int max_pages, const int32_t* old_len,
                               hipStream_t st) {
  const int W = n_runs * spr;
  hipLaunchKernelGGL(k_write_samples, dim3((W + 255) / 256), dim3(256), 0, st, c, n_runs, run_req,
                     run_start, run_len, spr, bt, max_pages, old_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_ensure(c, c.wneeded, W, c.wnofetch, nullptr, c.wmiss, c.wmiss_count, st);
  if (e != hipSuccess) return e;
  return launch_fetch(c, c.wmiss, c.wmiss_count, W, st);
}

// ---------------------------------------------------------- initialisation --
__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void k_fill_u8(uint8_t* p, int64_t n, uint8_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void k_iota_i32(int32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = (int32_t)i;
}
__global__ void k_reset_hdr(StateHdr* h) {
  if (threadIdx.x == 0) {
    h->clock = 0;
    for (int i = 0; i < CNT_N; ++i) h->counters[i] = 0;
    h->error_word = 0;
    h->parity = 0;
    h->pad[0] = h->pad[1] = 0;
  }
}

static hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int g = (int)((n + 255) / 256);
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(k_fill_i32, dim3(g), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_bytes(void* p, int64_t n, uint8_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int g = (int)((n + 255) / 256);
  if (g > 8192) g = 8192;
  hipLaunchKernelGGL(k_fill_u8, dim3(g), dim3(256), 0, st, (uint8_t*)p, n, v);
  return hipGetLastError();
}

// Empty pool, zero counters.  With full=1 also clear slab, running sums and
// the chain counters (first attach).
hipError_t launch_reset(const DevCtx& c, int full, hipStream_t st) {
  hipError_t e;
  if ((e = fill_i32(c.page_to_slot, c.N, -1, st)) != hipSuccess) return e;
  if ((e = fill_i32(c.page_mark, c.N, 0x7FFFFFFF, st)) != hipSuccess) return e;
  if ((e = fill_i32(c.slot_to_page, c.S, -1, st)) != hipSuccess) return e;
  if ((e = launch_fill_bytes(c.stamp, (int64_t)c.S * 8, 0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_iota_i32, dim3((c.S + 255) / 256), dim3(256), 0, st, c.order, (int64_t)c.S);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_reset_hdr, dim3(1), dim3(64), 0, st, c.hdr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (full) {
    const int64_t E = (int64_t)c.L * c.N * c.Hkv * c.D;
    if ((e = launch_fill_bytes(c.slab, E * 2, 0, st)) != hipSuccess) return e;
    if ((e = launch_fill_bytes(c.slab_acc, E * 8, 0, st)) != hipSuccess) return e;
    if ((e = fill_i32(c.row_done, c.max_rows, 0, st)) != hipSuccess) return e;
    if ((e = fill_i32(c.glob_done, 4, 0, st)) != hipSuccess) return e;
    if ((e = fill_i32(c.rest_ctr, 2, 0, st)) != hipSuccess) return e;
    if ((e = fill_i32(c.attn_done, (int64_t)c.max_batch * c.Hkv, 0, st)) != hipSuccess) return e;
    if ((e = fill_i32(reinterpret_cast<int32_t*>(c.sel_bm),
                      (int64_t)sel_bm_words(c.max_rows, c.max_batch, c.max_pages), 0, st)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(k_iota_i32, dim3((c.max_rows + 256) / 256), dim3(256), 0, st, c.iota, (int64_t)c.max_rows + 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------- codec hooks ----
__global__ void k_e4m3_encode(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (uint8_t)f32_to_e4m3(in[i]);
}
__global__ void k_e4m3_decode(const uint8_t* in, float* out, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    f32x2 v = e4m3x2_lo((uint32_t)in[i]);
    out[i] = v.x;
  }
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int g = (int)((n + 255) / 256);
  if (g > 8192) g = 8192;
  hipLaunchKernelGGL(k_e4m3_encode, dim3(g), dim3(256), 0, st, in, out, n);
  return hipGetLastError();
}
hipError_t launch_e4m3_decode(const uint8_t* in, float* out, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int g = (int)((n + 255) / 256);
  if (g > 8192) g = 8192;
  hipLaunchKernelGGL(k_e4m3_decode, dim3(g), dim3(256), 0, st, in, out, n);
  return hipGetLastError();
}
