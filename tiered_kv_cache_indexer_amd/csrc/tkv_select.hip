// Indexer top-k page selection and compact_selected_pages (gfx950).
//
// FreeToken PR #499, "Why this works for sparse attention": each attention
// step first scores the pages on a compressed key slab that stays on the GPU
// and keeps the top-k; "Design": compact_selected_pages caps the selection
// at max_sel_pages = 2*block_topk + 8 and counts what it drops.
//
// Decode launch: grid (chunks, rows), 256 threads.  Each workgroup scores
// CHUNK pages of one row: a wave reads one page's slab row (Hkv*d bf16 =
// 1 KiB at d=128, Hkv=4) with one 16-byte load per lane, multiplies by the
// per-group query sum held in registers and reduces across the lanes.  The
// last workgroup of a row (atomic counter) selects the row's top-k by radix
// select over the scores; the last row of the call compacts every request
// and, for the fused decode step, runs the LRU ensure in the same launch.
//
// Scores: a product of two bf16 values is exact in fp32; the products are
// summed in fp64, where every partial sum is exact as long as the page's
// products are multiples of 2^e with sum |q*slab| < 2^(53+e) (about 40 of
// the 53 bits for normally distributed bf16 queries and keys; 24 on the
// workloads' grids), so the score is the exact dot product rounded once to
// fp32 whatever the order of the additions -- and the selections are too.
#include "tkv_dev.h"
#include "tkv_launch.h"
#include "tkv_lru_dev.h"




__device__ __forceinline__ int request_of_row(const int32_t* row_start, int B, int r) {
  int b = 0;
  while (b + 1 < B && row_start[b + 1] <= r) ++b;
  return b;
}

__device__ __forceinline__ int visible_pages(const SelArgs& a, int PS, int b, int r) {
  int n = a.n_pages[b];
  n = n < a.max_pages ? n : a.max_pages;   // never past the block-table row
  if (n < 0) n = 0;
  if (a.row_pos) {
    int pos = a.row_pos[r];
    int v = pos < 0 ? 0 : pos / PS + 1;
    n = v < n ? v : n;
  }
  return n;
}

// Top-k of scores[0..visible) (ties -> lower index), ascending, -1 padded.
__device__ void row_topk_block(const float* scores, int visible, int k, int32_t* out,
                               uint32_t* keys, int* hist, int* sm_scan, int* sm_misc) {
  const int tid = threadIdx.x;
  if (visible <= k) {
    for (int j = tid; j < k; j += TKV_BLOCK) out[j] = j < visible ? j : -1;
    return;
  }
  for (int i = tid; i < visible; i += TKV_BLOCK) keys[i] = f32_order(scores[i]);
  uint32_t prefix = 0, mask = 0;
  int kk = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < visible; i += TKV_BLOCK) {
      uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    // suffix sums from the top digit down: thread t owns digit 255 - t
    int v = hist[255 - tid];
    int tot;
    int ex = block_excl_scan(v, &tot, sm_scan);
    int incl = ex + v;                           // keys with digit >= 255 - tid
    if (incl >= kk && ex < kk) {
      sm_misc[0] = 255 - tid;
      sm_misc[1] = ex;                           // keys with a strictly larger digit
    }
    __syncthreads();
    uint32_t d = (uint32_t)sm_misc[0];
    kk -= sm_misc[1];
    prefix |= d << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;                      // the k-th largest key; kk ties to take
  const int E = (visible + TKV_BLOCK - 1) / TKV_BLOCK;
  const int i0 = tid * E, i1 = min(visible, i0 + E);
  int ties = 0;
  for (int i = i0; i < i1; ++i) ties += keys[i] == T;
  int tot;
  int tie_base = block_excl_scan(ties, &tot, sm_scan);
  int nsel = 0;
  {
    int tr = tie_base;
    for (int i = i0; i < i1; ++i) {
      uint32_t key = keys[i];
      if (key > T) ++nsel;
      else if (key == T) { if (tr < kk) ++nsel; ++tr; }
    }
  }
  int out_base = block_excl_scan(nsel, &tot, sm_scan);
  {
    int tr = tie_base, pos = out_base;
    for (int i = i0; i < i1; ++i) {
      uint32_t key = keys[i];
      bool s = false;
      if (key > T) s = true;
      else if (key == T) { s = tr < kk; ++tr; }
      if (s) out[pos++] = i;
    }
  }
}

// Row top-k for k <= 64 (wave bitonic): each wave folds a share of the
// row's sorted 64-key lists into its running top-64 list (a merge per list
// that exists: 16 lists take 3 merges per wave, then 3 in wave 0), the four
// wave lists are merged through LDS, and wave 0 writes the first k indices
// ascending.  Measured on MI355X at 16 lists: 2.7 us from the last
// workgroup's arrival, where a one-wave radix descent over the lists' keys
// (up to 64 dependent ballot rounds) took 6.4 us.
// `load_list(c)` returns chunk c's sorted list in this lane.
template <typename LoadList>
__device__ void row_topk64_block(int n_lists, int k, int32_t* out, uint64_t* lds64, LoadList load_list) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int BATCH = 16;  // lists loaded per wave before merging (loads in flight together)
  uint64_t run = 0;
  for (int base = wave; base < n_lists; base += 4 * BATCH) {
    uint64_t v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = base + 4 * u;
      v[u] = c < n_lists ? load_list(c) : 0ull;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (base + 4 * u >= n_lists) break;           // wave-uniform: no merges with empty lists
      run = (base == wave && u == 0) ? v[u] : wave_merge_desc(run, v[u]);
    }
  }
  lds64[wave * 64 + lane] = run;
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < 4 && w < n_lists; ++w) run = wave_merge_desc(run, lds64[w * 64 + lane]);
    int idx = (lane < k && run != 0) ? sel_key_index(run) : 0x7FFFFFFF;
    idx = wave_sort_asc_i32(idx);
    if (lane < k) out[lane] = idx == 0x7FFFFFFF ? -1 : idx;
  }
  __syncthreads();
}

// Union of request b's rows, ascending, unique; first C kept, rest counted.
// Bitmap group of row r of request b: each request's rows are cut into groups
// of 64, the groups of earlier requests first.
__device__ __forceinline__ int sel_bm_group(const SelArgs& a, int b, int r) {
  int g = 0;
  for (int bb = 0; bb < b; ++bb) g += (a.row_start[bb + 1] - a.row_start[bb] + 63) >> 6;
  return g + ((r - a.row_start[b]) >> 6);
}

// Called by the whole block once row r's selection is written: marks its pages
// in its group's bitmap (requests with several rows only), so that the union
// is a few bitmaps to OR instead of every row's list to re-read.
__device__ void mark_row_pages(const DevCtx& c, const SelArgs& a, int b, int r) {
  if (a.row_start[b + 1] - a.row_start[b] <= 1) return;
  __syncthreads();
  const int words = (a.max_pages + 31) >> 5;
  uint32_t* bm = c.sel_bm + (size_t)sel_bm_group(a, b, r) * words;
  for (int j = threadIdx.x; j < a.topk; j += TKV_BLOCK) {
    const int i = a.sel_local[(size_t)r * a.topk + j];
    if (i >= 0 && i < a.max_pages) atomicOr(&bm[i >> 5], 1u << (i & 31));
  }
}

// Union of a multi-row request's selections: OR of its group bitmaps (which
// are cleared again), ascending local ids, first C kept, the rest counted as
// drops, translated through the block table.
__device__ void compact_block(const DevCtx& c, const SelArgs& a, int b, uint32_t* bm, int* sm_scan) {
  const int tid = threadIdx.x;
  const int words = (a.max_pages + 31) >> 5;
  for (int w = tid; w < words; w += TKV_BLOCK) bm[w] = 0;
  __syncthreads();
  const int r0 = a.row_start[b], r1 = a.row_start[b + 1];
  const int ng = (r1 - r0 + 63) >> 6;
  uint32_t* gbm = c.sel_bm + (size_t)sel_bm_group(a, b, r0) * words;
  const int tot = ng * words;
  constexpr int U = 8;
  for (int base = 0; base < tot; base += TKV_BLOCK * U) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * TKV_BLOCK + tid;
      v[u] = idx < tot ? gbm[idx] : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * TKV_BLOCK + tid;
      if (idx < tot) {
        if (v[u]) atomicOr(&bm[idx % words], v[u]);
        gbm[idx] = 0u;
      }
    }
  }
  __syncthreads();
  const int WPT = (words + TKV_BLOCK - 1) / TKV_BLOCK;
  const int w0 = tid * WPT, w1 = min(words, w0 + WPT);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  int u;
  int pos = block_excl_scan(cnt, &u, sm_scan);
  int32_t* nd = a.needed + (size_t)b * a.C;
  const int32_t* btb = a.bt + (size_t)b * a.max_pages;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bm[w];
    while (bits) {
      int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < a.C) nd[pos] = btb[(w << 5) + bit];
      ++pos;
    }
  }
  for (int p = u + tid; p < a.C; p += TKV_BLOCK) nd[p] = -1;
  if (tid == 0 && u > a.C) c.hdr->counters[CNT_DROPS] += u - a.C;
  __syncthreads();
}

// Slots of every row's selected pages, all rows in one pass (one round trip
// to memory for any batch): a row that is its request's only row with top-k
// <= C takes them from the ensure's output (its selection is the needed list,
// in order); other rows translate page -> slot after the ensure.
__device__ void write_sel_slots(const DevCtx& c, const SelArgs& a) {
  const int n = a.rows * a.topk;
  for (int e = threadIdx.x; e < n; e += TKV_BLOCK) {
    const int r = e / a.topk, j = e - r * a.topk;
    const int b = request_of_row(a.row_start, a.B, r);
    const int i = a.sel_local[e];
    int slot = -1;
    if (i >= 0 && i < a.max_pages) {
      if (a.row_start[b + 1] - a.row_start[b] == 1 && a.topk <= a.C) {
        slot = a.out_slots[(size_t)b * a.C + j];
      } else {
        const int p = a.bt[(size_t)b * a.max_pages + i];
        if (p >= 0 && (int64_t)p < c.N) slot = c.page_to_slot[p];
      }
    }
    a.sel_slots[e] = slot;
  }
}

// Shared tail once every row's selection is written: compaction and ensure.
// Requests with one row, all in one pass (one round trip for the selections
// and one for the block table, whatever the batch): such a row's selection
// is already ascending and unique, so its compaction is a block-table lookup
// of the first C entries, and each valid entry past C is a drop.
__device__ void compact_single_rows(const DevCtx& c, const SelArgs& a, int* sm_scan) {
  const int J = a.topk > a.C ? a.topk : a.C;
  int drops = 0;
  for (int e = threadIdx.x; e < a.B * J; e += TKV_BLOCK) {
    const int b = e / J, j = e - b * J;
    const int r = a.row_start[b];
    if (a.row_start[b + 1] - r != 1) continue;
    const int i = j < a.topk ? a.sel_local[(size_t)r * a.topk + j] : -1;
    if (j < a.C) {
      int v = -1;
      if (i >= 0 && i < a.max_pages) v = a.bt[(size_t)b * a.max_pages + i];
      a.needed[(size_t)b * a.C + j] = v;
    } else if (i >= 0) {
      ++drops;
    }
  }
  drops = block_sum(drops, sm_scan);
  if (threadIdx.x == 0 && drops > 0) c.hdr->counters[CNT_DROPS] += drops;
  __syncthreads();
}

// One request with one row r, in the row's last workgroup: the batch's rows
// compact in parallel, ahead of the call's tail.
__device__ void compact_one_row(const DevCtx& c, const SelArgs& a, int b, int r, int* sm_scan) {
  __syncthreads();                                          // the row's selection is written
  const int J = a.topk > a.C ? a.topk : a.C;
  int drops = 0;
  for (int j = threadIdx.x; j < J; j += TKV_BLOCK) {
    const int i = j < a.topk ? a.sel_local[(size_t)r * a.topk + j] : -1;
    if (j < a.C) {
      int v = -1;
      if (i >= 0 && i < a.max_pages) v = a.bt[(size_t)b * a.max_pages + i];
      a.needed[(size_t)b * a.C + j] = v;
    } else if (i >= 0) {
      ++drops;
    }
  }
  drops = block_sum(drops, sm_scan);
  if (threadIdx.x == 0 && drops > 0)
    atomicAdd(reinterpret_cast<unsigned long long*>(&c.hdr->counters[CNT_DROPS]), (unsigned long long)drops);
  __syncthreads();
}

// `rows_compacted`: the one-row requests were compacted by their rows' last
// workgroups.
__device__ void select_finish(const DevCtx& c, const SelArgs& a, uint32_t* dyn, int* sm_scan,
                              bool rows_compacted) {
  if (!rows_compacted) compact_single_rows(c, a, sm_scan);
  if (!a.one_row_each)
    for (int b = 0; b < a.B; ++b)
      if (a.row_start[b + 1] - a.row_start[b] != 1) compact_block(c, a, b, dyn, sm_scan);
  if (a.do_ensure) {
    EnsureOut o{a.out_slots, a.miss, a.miss_count, a.miss_flag};
    lru_ensure_block(c, a.needed, a.B * a.C, nullptr, o, sm_scan, dyn);   // dyn is free after the compaction
    __syncthreads();
    if (a.sel_slots) write_sel_slots(c, a);
  }
}

template <int E8>
__global__ __launch_bounds__(TKV_BLOCK) void k_select_scan(DevCtx c, SelArgs a) {
  extern __shared__ __align__(16) uint32_t dyn[];
  __shared__ int hist[256];
  __shared__ int sm_scan[8];
  __shared__ int sm_misc[8];
  __shared__ int sm_b;
  __shared__ uint64_t sm_keys[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.y, chunk = blockIdx.x;
  constexpr int G = 8;                                // query heads per KV head (validated on the host)
  constexpr int E = E8 * 8;                           // Hkv * D
  constexpr int PPW = E8 >= 64 ? 1 : 64 / E8;         // pages per wave pass
  constexpr int SPL = E8 >= 64 ? E8 / 64 : 1;         // 16-byte segments per lane
  constexpr int LANES = E8 >= 64 ? 64 : E8;           // lanes per page
  constexpr int PASSES = SEL_CHUNK / 4 / PPW;         // wave passes per chunk
  // (decode calls: row r is request r, no lookup before the loads below)
  if (tid == 0 && !a.one_row_each) sm_b = request_of_row(a.row_start, a.B, r);
  __syncthreads();
  const int b = a.one_row_each ? r : sm_b;
  const int p_begin = chunk * SEL_CHUNK;
  const int32_t* btb = a.bt + (size_t)b * a.max_pages;
  const int sub = lane / LANES, seg0 = lane % LANES;

  // block-table entries first, up to the row's end (not the visible count,
  // whose load they would otherwise wait for): independent of the query sums
  const int p_lim = min(a.max_pages, p_begin + SEL_CHUNK);
  int logical[PASSES];
#pragma unroll
  for (int it = 0; it < PASSES; ++it) {
    const int p = p_begin + (it * 4 + wave) * PPW + sub;
    int lg = -1;
    if (p < p_lim) lg = btb[p];
    logical[it] = lg;
  }
  // the query rows of the lane's 8-element segments (element e0 = 8 * segment:
  // group e0 / d, dims e0 % d .. +7), one 16-byte load per group head; each
  // wave forms its own group sums, so nothing waits at a barrier and the
  // slab loads below are in flight while they are summed
  uint4 qraw[SPL][G];
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int e0 = (seg0 + s * 64) * 8, g = e0 / c.D;
    const uint16_t* qp = a.q + ((size_t)r * c.Hq + g * G) * c.D + (e0 - g * c.D);
#pragma unroll
    for (int h = 0; h < G; ++h) qraw[s][h] = *reinterpret_cast<const uint4*>(qp + (size_t)h * c.D);
  }
  const int visible = visible_pages(a, c.PS, b, r);
  const int p_end = min(visible, p_begin + SEL_CHUNK);
#pragma unroll
  for (int it = 0; it < PASSES; ++it) {
    const int p = p_begin + (it * 4 + wave) * PPW + sub;
    const int lg = logical[it];
    logical[it] = (p < p_end && (int64_t)lg >= 0 && (int64_t)lg < c.N) ? lg : -1;
  }
  const uint16_t* slab_l = c.slab + (size_t)a.layer * c.N * E;
  uint4 v[PASSES][SPL];
#pragma unroll
  for (int it = 0; it < PASSES; ++it)
#pragma unroll
    for (int s = 0; s < SPL; ++s)
      v[it][s] = logical[it] >= 0
                     ? reinterpret_cast<const uint4*>(slab_l + (size_t)logical[it] * E)[seg0 + s * 64]
                     : make_uint4(0, 0, 0, 0);
  // per-group query sum: exact (fp64) sum of the group's 8 bf16 heads -> fp32 -> bf16
  float qg[SPL][8];
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      double acc = 0.0;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t w = (&qraw[s][h].x)[t >> 1];
        acc += (double)__uint_as_float((t & 1) ? (w & 0xFFFF0000u) : (w << 16));
      }
      qg[s][t] = bf16_to_f32(f32_to_bf16((float)acc));
    }
  }
  float keys[PASSES];
#pragma unroll
  for (int it = 0; it < PASSES; ++it) {
    double part = 0.0;
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      const uint32_t w[4] = {v[it][s].x, v[it][s].y, v[it][s].z, v[it][s].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        part += (double)(qg[s][2 * t] * __uint_as_float(w[t] << 16));            // exact product
        part += (double)(qg[s][2 * t + 1] * __uint_as_float(w[t] & 0xFFFF0000u));
      }
    }
#pragma unroll
    for (int o = LANES / 2; o > 0; o >>= 1) part += xor_lane_f64(part, o);
    const int lg = logical[it];
    float key = (float)part;
    if (lg < 0) key = -INFINITY;
    else if (a.bias) key = key + a.bias[lg];
    keys[it] = key;
  }
  float* sc = c.scores + (size_t)r * c.max_pages;
  uint64_t* cand = reinterpret_cast<uint64_t*>(c.scores) + (size_t)r * a.n_chunks * 64;
  if (a.topk <= 64) {
    // this chunk's 64 pages as one sorted list
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int p = p_begin + (it * 4 + wave) * PPW + sub;
      if (seg0 == 0) sm_keys[p - p_begin] = (p < p_end) ? sel_key(keys[it], p) : 0ull;
    }
    __syncthreads();
    if (wave == 0) cand[(size_t)chunk * 64 + lane] = wave_sort_desc(sm_keys[lane]);
  } else {
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int p = p_begin + (it * 4 + wave) * PPW + sub;
      if (p < p_end && seg0 == 0) sc[p] = keys[it];
    }
  }
  if (!last_block_arrive(&c.row_done[r], a.n_chunks, &sm_misc[4])) return;
  int32_t* out_r = a.sel_local + (size_t)r * a.topk;
  if (a.topk <= 64) {
    row_topk64_block(a.n_chunks, a.topk, out_r, reinterpret_cast<uint64_t*>(dyn),
                     [&](int ch) { return cand[(size_t)ch * 64 + lane]; });
  } else {
    row_topk_block(sc, visible, a.topk, out_r, dyn, hist, sm_scan, sm_misc);
  }
  if (a.one_row_each || a.row_start[b + 1] - a.row_start[b] == 1) {
    compact_one_row(c, a, b, r, sm_scan);
  } else {
    mark_row_pages(c, a, b, r);
  }
  // a single row's last workgroup is the last workgroup of the launch
  if (a.rows > 1 && !last_block_arrive(&c.glob_done[0], a.rows, &sm_misc[2])) return;
  select_finish(c, a, dyn, sm_scan, true);
}

// Tail-only launch: scores already in the workspace (prefill scoring kernel).
// One workgroup per row; the union and compaction run in k_select_finish
// after it.  With thousands of rows a last-workgroup hand-off would cost every
// workgroup an L2 write-back (the release between XCDs); the kernel boundary
// pays it once.
__global__ __launch_bounds__(TKV_BLOCK) void k_select_rows(DevCtx c, SelArgs a) {
  extern __shared__ __align__(16) uint32_t dyn[];
  __shared__ int hist[256];
  __shared__ int sm_scan[8];
  __shared__ int sm_misc[8];
  __shared__ int sm_b;
  const int r = blockIdx.x, lane = threadIdx.x & 63;
  if (threadIdx.x == 0) sm_b = request_of_row(a.row_start, a.B, r);
  __syncthreads();
  const int b = sm_b;
  const int visible = visible_pages(a, c.PS, b, r);
  const float* sc = c.scores + (size_t)r * c.max_pages;
  if (a.topk <= 64) {
    const int n_lists = (visible + 63) / 64;
    row_topk64_block(n_lists, a.topk, a.sel_local + (size_t)r * a.topk, reinterpret_cast<uint64_t*>(dyn),
                     [&](int ch) {
                       const int p = ch * 64 + lane;
                       return wave_sort_desc(p < visible ? sel_key(sc[p], p) : 0ull);
                     });
  } else {
    row_topk_block(sc, visible, a.topk, a.sel_local + (size_t)r * a.topk, dyn, hist, sm_scan, sm_misc);
  }
  mark_row_pages(c, a, b, r);
}

// Wave count of a per-lane count below 2^6: one ballot per bit.
__device__ __forceinline__ int wave_count6(int cnt) {
  int tot = 0;
#pragma unroll
  for (int j = 0; j < 6; ++j) tot += __popcll(__ballot((cnt >> j) & 1)) << j;
  return tot;
}

// One wave per row, keys of up to 64*NPL visible pages in registers.  The
// k-th largest key T is the k-th of the few keys at or above a bound taken
// from the lanes' maxima (below); where those are more than 64, T is found by
// a radix descent from the top bit: a bit is kept when at least k keys are
// >= the prefix with it set, and the descent stops early once exactly k keys
// are >= the prefix.  Keys are unique (the
// low word is ~page), so exactly min(k, visible) keys are >= T; they are
// written in ascending page order by ballot prefix counts.
// Workgroup size of the per-row top-k: 4 rows (16 measured the same).
#define RW_BLOCK TKV_BLOCK

// Nonzero words of the LDS group bitmap into the global one (the group of
// the workgroup's first wave).
template <int NW_WORDS>
__device__ __forceinline__ void rows_wave_flush(const DevCtx& c, const uint32_t* wbm, const int* wgrp, int words) {
  const int g0 = wgrp[0];
  if (g0 < 0) return;
  for (int w = threadIdx.x; w < NW_WORDS && w < words; w += RW_BLOCK)
    if (wbm[w]) atomicOr(&c.sel_bm[(size_t)g0 * words + w], wbm[w]);
}

template <int NPL>
__global__ __launch_bounds__(RW_BLOCK) void k_select_rows_wave(DevCtx c, SelArgs a) {
  constexpr int NW = RW_BLOCK / 64;
  __shared__ uint64_t cbuf[NW][64];
  __shared__ uint32_t wbm[2 * NPL];   // the first wave's group bitmap (64 * NPL pages)
  __shared__ int wgrp[NW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * NW + wave;
  for (int w = threadIdx.x; w < 2 * NPL; w += RW_BLOCK) wbm[w] = 0u;
  const int words = (a.max_pages + 31) >> 5;   // <= 2 * NPL (max_pages <= 64 * NPL)
  if (r >= a.rows) {
    if (lane == 0) wgrp[wave] = -1;
    __syncthreads();
    __syncthreads();
    rows_wave_flush<2 * NPL>(c, wbm, wgrp, words);
    return;
  }
  const int b = request_of_row(a.row_start, a.B, r);
  const int visible = visible_pages(a, c.PS, b, r);
  const float* sc = c.scores + (size_t)r * c.max_pages;
  // keys stay in registers: every load is in bounds (index clamped) and every
  // loop below is fully unrolled without data-dependent branches; keys past
  // the visible pages are 0, which no threshold (>= 1) counts
  uint64_t key[NPL];
  const int pmax = visible > 0 ? visible - 1 : 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int p = i * 64 + lane;
    const float v = sc[min(p, pmax)];
    key[i] = p < visible ? sel_key(v, p) : 0ull;   // valid keys are nonzero
  }
  const int k = a.topk;
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t thr = 1;
  bool found = visible <= k;
  if (!found && k <= 64) {
    // A bound from the lanes' maxima: the k-th largest of them, T, has at
    // least k keys at or above it, so the k-th largest key is >= T.  The keys
    // >= T (about 43 of 1,088 random keys for k = 32, more than 64 in about
    // 1 of 20,000 rows) are gathered and sorted in one wave; the k-th of
    // them is the threshold.  With more than 64 the radix descent decides.
    uint64_t lm = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) lm = key[i] > lm ? key[i] : lm;
    const uint64_t T = shfl_u64(wave_sort_desc(lm), k - 1);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) cnt += key[i] >= T ? 1 : 0;
    if (wave_count6(cnt) <= 64) {
      uint64_t* cb = cbuf[threadIdx.x >> 6];
      int base = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const bool s = key[i] >= T;
        const uint64_t m = __ballot(s);
        if (s) cb[base + __popcll(m & below)] = key[i];
        base += __popcll(m);
      }
      __builtin_amdgcn_s_waitcnt(0);
      const uint64_t cv = lane < base ? cb[lane] : 0ull;
      thr = shfl_u64(wave_sort_desc(cv), k - 1);
      found = true;
    }
  }
  if (!found) {
    uint64_t t = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = t | (1ull << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) cnt += key[i] >= cand ? 1 : 0;
      const int tot = wave_count6(cnt);
      if (tot >= k) {
        t = cand;
        if (tot == k) break;
      }
    }
    thr = t;
  }
  int32_t* out = a.sel_local + (size_t)r * k;
  // a request with several rows marks the row's pages in its group's bitmap:
  // the waves whose group is the first wave's OR into LDS (the workgroup's
  // rows are consecutive, so normally all of them) and the workgroup flushes
  // each nonzero word with one atomic; other waves mark the global bitmap
  const bool multi = a.row_start[b + 1] - a.row_start[b] > 1;
  const int grp = multi ? sel_bm_group(a, b, r) : -1;
  if (lane == 0) wgrp[wave] = grp;
  __syncthreads();
  const bool to_lds = grp >= 0 && grp == wgrp[0];
  uint32_t* bm = (grp >= 0 && !to_lds) ? c.sel_bm + (size_t)grp * words : nullptr;
  int base = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool s = key[i] >= thr;
    const uint64_t m = __ballot(s);
    if (s) {
      const int p = i * 64 + lane;
      out[base + __popcll(m & below)] = p;
      if (to_lds) atomicOr(&wbm[p >> 5], 1u << (p & 31));
      else if (bm) atomicOr(&bm[p >> 5], 1u << (p & 31));
    }
    base += __popcll(m);
  }
  for (int j = base + lane; j < k; j += 64) out[j] = -1;
  __syncthreads();
  rows_wave_flush<2 * NPL>(c, wbm, wgrp, words);
}

__global__ __launch_bounds__(TKV_BLOCK) void k_select_finish(DevCtx c, SelArgs a) {
  extern __shared__ __align__(16) uint32_t dyn[];
  __shared__ int sm_scan[8];
  select_finish(c, a, dyn, sm_scan, false);
}

__global__ __launch_bounds__(TKV_BLOCK) void k_ensure(DevCtx c, const int32_t* needed, int W,
                                                      const uint8_t* no_fetch, EnsureOut o) {
  extern __shared__ __align__(16) uint32_t dyn[];
  __shared__ int sm_scan[8];
  lru_ensure_block(c, needed, W, no_fetch, o, sm_scan, dyn);
}

// ------------------------------------------------------------------ launchers --
static size_t ensure_dyn_lds(const DevCtx& c) { return lru_lds_words(c.S) * 4; }

size_t select_dyn_lds(const DevCtx& c) {
  size_t keys = (size_t)c.max_pages * 4;
  size_t bm = (size_t)((c.max_pages + 31) / 32) * 4;
  size_t lists = 4 * 64 * 8;
  size_t m = keys > bm ? keys : bm;
  m = m > lists ? m : lists;
  return m > ensure_dyn_lds(c) ? m : ensure_dyn_lds(c);
}

hipError_t launch_select_scan(const DevCtx& c, const SelArgs& a, hipStream_t st) {
  dim3 grid(a.n_chunks, a.rows);
  size_t lds = select_dyn_lds(c);
  const int E8 = c.Hkv * c.D / 8;
  if (E8 == 64) hipLaunchKernelGGL(k_select_scan<64>, grid, dim3(TKV_BLOCK), lds, st, c, a);
  else if (E8 == 16) hipLaunchKernelGGL(k_select_scan<16>, grid, dim3(TKV_BLOCK), lds, st, c, a);
  else if (E8 == 32) hipLaunchKernelGGL(k_select_scan<32>, grid, dim3(TKV_BLOCK), lds, st, c, a);
  else if (E8 == 128) hipLaunchKernelGGL(k_select_scan<128>, grid, dim3(TKV_BLOCK), lds, st, c, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_select_rows(const DevCtx& c, const SelArgs& a, hipStream_t st) {
  const dim3 wgrid((a.rows + RW_BLOCK / 64 - 1) / (RW_BLOCK / 64));
  if (a.max_pages <= 512) hipLaunchKernelGGL(k_select_rows_wave<8>, wgrid, dim3(RW_BLOCK), 0, st, c, a);
  else if (a.max_pages <= 1024) hipLaunchKernelGGL(k_select_rows_wave<16>, wgrid, dim3(RW_BLOCK), 0, st, c, a);
  else if (a.max_pages <= 1536) hipLaunchKernelGGL(k_select_rows_wave<24>, wgrid, dim3(RW_BLOCK), 0, st, c, a);
  else if (a.max_pages <= 2048) hipLaunchKernelGGL(k_select_rows_wave<32>, wgrid, dim3(RW_BLOCK), 0, st, c, a);
  else hipLaunchKernelGGL(k_select_rows, dim3(a.rows), dim3(TKV_BLOCK), select_dyn_lds(c), st, c, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select_finish, dim3(1), dim3(TKV_BLOCK), select_dyn_lds(c), st, c, a);
  return hipGetLastError();
}

hipError_t launch_ensure(const DevCtx& c, const int32_t* needed, int W, const uint8_t* no_fetch,
                         int32_t* out_slots, int32_t* miss, int32_t* miss_count, hipStream_t st) {
  EnsureOut o{out_slots, miss, miss_count, nullptr};
  hipLaunchKernelGGL(k_ensure, dim3(1), dim3(TKV_BLOCK), ensure_dyn_lds(c), st, c, needed, W, no_fetch, o);
  return hipGetLastError();
}
