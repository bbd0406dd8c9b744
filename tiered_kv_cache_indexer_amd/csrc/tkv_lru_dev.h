// Device-side LRU ensure, run by one 256-thread workgroup.
//
// FreeToken PR #499 ("What", "Design"): the GPU pool is an LRU cache of
// physical slots over the logical page space; the ensure is device-side and
// fixed-shape; the mirror is write-through, so evicting a page only rebinds
// its slot.  Policy (one clock tick per call): distinct needed pages in
// first-occurrence order; resident pages are hits and get the new stamp; the
// misses, in first-occurrence order, take the slots not hit by this call in
// ascending (stamp, slot) order.
//
// The (stamp, slot) order is kept incrementally in `order[parity]`: slots not
// touched by a call keep their relative order and every touched slot gets the
// newest stamp, so the next order is "untouched slots in old order, then the
// touched slots by index".  Victims are the first M untouched entries.  Each
// step is a block-wide scan over the needed list or over the slots, so a call
// costs O(width + slots) with no sort.
#pragma once
#include "tkv_dev.h"

#define LRU_CH 8   // order entries per thread per pass

struct EnsureOut {
  int32_t* out_slots;   // [W] or null
  int32_t* miss;        // [W][2]
  int32_t* miss_count;  // [1]
  uint8_t* miss_flag;   // [W] or null: 1 where the entry's page is on this call's fetch list
                        // (a duplicate takes its first occurrence's flag), else 0
};

__device__ __forceinline__ bool page_ok(const DevCtx& c, int p) { return p >= 0 && (int64_t)p < c.N; }

// `tb`: LDS bitset of the slots touched by this call (hit or bound), at
// least (S + 31) / 32 words; it lives only for the call.
__device__ __forceinline__ bool slot_touched(const uint32_t* tb, int s) { return (tb[s >> 5] >> (s & 31)) & 1u; }
__device__ __forceinline__ void touch_slot(uint32_t* tb, int s) { atomicOr(&tb[s >> 5], 1u << (s & 31)); }

__device__ void lru_ensure_global(const DevCtx& c, const int32_t* needed, int W,
                                  const uint8_t* no_fetch, EnsureOut o, int* sm_scan, uint32_t* tb) {
  const int tid = threadIdx.x;
  const int32_t INTMAX = 0x7FFFFFFF;
  for (int w = tid; w < (c.S + 31) >> 5; w += TKV_BLOCK) tb[w] = 0u;

  // A: first occurrence of every valid page id (atomicMin of the index)
  int bad = 0;
  for (int j = tid; j < W; j += TKV_BLOCK) {
    int p = needed[j];
    if (p == -1) continue;
    if (!page_ok(c, p)) { bad = 1; continue; }
    atomicMin(&c.page_mark[p], j);
  }
  if (bad) set_error(c.hdr, DERR_PAGE_RANGE);
  __syncthreads();

  // B: distinct pages; the capacity check precedes any state change
  int local = 0;
  for (int j = tid; j < W; j += TKV_BLOCK) {
    int p = needed[j];
    if (page_ok(c, p) && ld_acquire_i32(&c.page_mark[p]) == j) ++local;
  }
  const int distinct = block_sum(local, sm_scan);
  const int par = c.hdr->parity;
  const int64_t clock_new = c.hdr->clock + 1;

  if (distinct > c.S) {
    for (int j = tid; j < W; j += TKV_BLOCK) {
      int p = needed[j];
      if (page_ok(c, p)) c.page_mark[p] = INTMAX;
      if (o.out_slots) o.out_slots[j] = -1;
    }
    if (tid == 0) {
      set_error(c.hdr, DERR_CAPACITY);
      *o.miss_count = 0;
    }
    return;
  }

  // C: hits are restamped; misses are ranked in first-occurrence order
  int n_hits = 0;
  int M = 0;
  for (int base = 0; base < W; base += TKV_BLOCK) {
    int j = base + tid;
    int is_miss = 0;
    if (j < W) {
      int p = needed[j];
      if (page_ok(c, p) && ld_acquire_i32(&c.page_mark[p]) == j) {
        int s = c.page_to_slot[p];
        if (s >= 0) {
          touch_slot(tb, s);
          c.stamp[s] = clock_new;
          c.slot_of_j[j] = s;
          ++n_hits;
        } else {
          is_miss = 1;
        }
        if (o.miss_flag) o.miss_flag[j] = (is_miss && !(no_fetch && no_fetch[j])) ? 1 : 0;
      }
    }
    int tot;
    int ex = block_excl_scan(is_miss, &tot, sm_scan);
    if (is_miss) c.miss_j[M + ex] = j;
    M += tot;
  }
  __syncthreads();

  // D: victims = the first M slots of the (stamp, slot) order not hit here.
  // Each thread owns ch = ceil(S / 256) (at most LRU_CH) consecutive order
  // entries, so a pass over up to 256 * LRU_CH slots is one round of loads
  // and one block scan (ranks stay in order: earlier threads own earlier
  // entries).
  const int ch = min(LRU_CH, (c.S + TKV_BLOCK - 1) / TKV_BLOCK);   // entries per thread
  {
    int got = 0;
    const int32_t* ord = c.order + (size_t)par * c.S;
    for (int base = 0; base < c.S && got < M; base += TKV_BLOCK * ch) {
      const int i0 = base + tid * ch;
      int sl[LRU_CH], cand[LRU_CH];
#pragma unroll
      for (int u = 0; u < LRU_CH; ++u) sl[u] = (u < ch && i0 + u < c.S) ? ord[i0 + u] : 0;
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < LRU_CH; ++u) {
        cand[u] = (u < ch && i0 + u < c.S) && !slot_touched(tb, sl[u]);
        cnt += cand[u];
      }
      int tot;
      int r = got + block_excl_scan(cnt, &tot, sm_scan);
#pragma unroll
      for (int u = 0; u < LRU_CH; ++u)
        if (cand[u]) {
          if (r < M) c.victims[r] = sl[u];
          ++r;
        }
      got += tot;
    }
  }
  __syncthreads();

  // E: bind each miss to its victim (an evicted page just loses its slot)
  int n_evict = 0;
  for (int m = tid; m < M; m += TKV_BLOCK) {
    int j = c.miss_j[m];
    int p = needed[j];
    int s = c.victims[m];
    int old = c.slot_to_page[s];
    if (old >= 0) {
      c.page_to_slot[old] = -1;
      ++n_evict;
    }
    c.page_to_slot[p] = s;
    c.slot_to_page[s] = p;
    c.stamp[s] = clock_new;
    touch_slot(tb, s);
    c.slot_of_j[j] = s;
  }
  __syncthreads();

  // fetch list: misses not marked no_fetch, in first-occurrence order
  int MF = 0;
  for (int base = 0; base < M; base += TKV_BLOCK) {
    int m = base + tid;
    int f = 0, j = 0;
    if (m < M) {
      j = c.miss_j[m];
      f = (no_fetch && no_fetch[j]) ? 0 : 1;
    }
    int tot;
    int ex = block_excl_scan(f, &tot, sm_scan);
    if (f) {
      o.miss[2 * (MF + ex)] = c.slot_of_j[j];
      o.miss[2 * (MF + ex) + 1] = needed[j];
    }
    MF += tot;
  }

  // F: out_slots and fetch flags (a duplicate reads its first occurrence's)
  for (int j = tid; j < W; j += TKV_BLOCK) {
    int p = needed[j];
    int s = -1, f = 0;
    bool first = false;
    if (page_ok(c, p)) {
      const int j0 = ld_acquire_i32(&c.page_mark[p]);
      s = c.slot_of_j[j0];
      first = j0 == j;                         // its flag was written in C
      if (o.miss_flag && !first) f = o.miss_flag[j0];
    }
    if (o.out_slots) o.out_slots[j] = s;
    if (o.miss_flag && !first) o.miss_flag[j] = f;
  }
  __syncthreads();
  // G: release the first-occurrence marks
  for (int j = tid; j < W; j += TKV_BLOCK) {
    int p = needed[j];
    if (page_ok(c, p)) c.page_mark[p] = INTMAX;
  }

  // H: next order = untouched slots in old order, then touched slots by index
  // (ch consecutive entries per thread per pass, as in D)
  {
    const int32_t* ord = c.order + (size_t)par * c.S;
    int32_t* nxt = c.order + (size_t)(1 - par) * c.S;
    int run = 0;
    for (int base = 0; base < c.S; base += TKV_BLOCK * ch) {
      const int i0 = base + tid * ch;
      int sl[LRU_CH], keep[LRU_CH];
#pragma unroll
      for (int u = 0; u < LRU_CH; ++u) sl[u] = (u < ch && i0 + u < c.S) ? ord[i0 + u] : 0;
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < LRU_CH; ++u) {
        keep[u] = (u < ch && i0 + u < c.S) && !slot_touched(tb, sl[u]);
        cnt += keep[u];
      }
      int tot;
      int r = run + block_excl_scan(cnt, &tot, sm_scan);
#pragma unroll
      for (int u = 0; u < LRU_CH; ++u)
        if (keep[u]) nxt[r++] = sl[u];
      run += tot;
    }
    __syncthreads();
    for (int base = 0; base < c.S; base += TKV_BLOCK * ch) {
      const int s0 = base + tid * ch;
      int t[LRU_CH];
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < LRU_CH; ++u) {
        t[u] = (u < ch && s0 + u < c.S) ? (int)slot_touched(tb, s0 + u) : 0;
        cnt += t[u];
      }
      int tot;
      int r = run + block_excl_scan(cnt, &tot, sm_scan);
#pragma unroll
      for (int u = 0; u < LRU_CH; ++u)
        if (t[u]) nxt[r++] = s0 + u;
      run += tot;
    }
  }

  // I: clock, parity, counters
  int hits = block_sum(n_hits, sm_scan);
  int ev = block_sum(n_evict, sm_scan);
  if (tid == 0) {
    StateHdr* h = c.hdr;
    h->clock = clock_new;
    h->parity = 1 - par;
    h->counters[CNT_ENSURE] += 1;
    h->counters[CNT_HITS] += hits;
    h->counters[CNT_MISSES] += MF;
    h->counters[CNT_FRESH] += M - MF;
    h->counters[CNT_EVICT] += ev;
    *o.miss_count = MF;
  }
}

// ---- LDS path: widths up to LRU_LDS_W, pools up to TKV_BLOCK * LRU_CH slots ----
// The same policy with every read of the residency state issued at the start
// (the header, the needed ids and their slots, this thread's order entries
// and the pages their slots hold), so the phases below wait on LDS and block
// scans only.  First occurrences come from an LDS hash table (page -> least
// index, linear probing) instead of the global page marks.  Measured on
// MI355X, the global path spends most of its time in dependent round trips
// to state written by earlier kernels (each one a miss in this XCD's L2).
#define LRU_LDS_W 512    // widths served from LDS
#define LRU_HT 1024      // hash slots (>= 2 * LRU_LDS_W)
#define LRU_HT_EMPTY (-1)

__host__ __device__ inline int lru_lds_fast_ok(int S) { return S <= TKV_BLOCK * LRU_CH; }
// 32-bit words of dynamic LDS the ensure needs: the touched-slot bitset, and
// with the LDS path the hash table and five [LRU_LDS_W] lists
__host__ __device__ inline size_t lru_lds_words(int S) {
  const size_t tbw = (size_t)((S + 31) >> 5);
  return lru_lds_fast_ok(S) ? tbw + 2 * LRU_HT + 5 * LRU_LDS_W : tbw;
}

__device__ __forceinline__ int lru_hash(int p) { return (int)(((uint32_t)p * 2654435761u) >> 22); }   // 10 bits

__device__ void lru_ensure_lds(const DevCtx& c, const int32_t* needed, int W, const uint8_t* no_fetch,
                               EnsureOut o, int* sm_scan, uint32_t* dyn) {
  constexpr int JPT = LRU_LDS_W / TKV_BLOCK;   // needed entries per thread
  const int tid = threadIdx.x;
  const int S = c.S, tbw = (S + 31) >> 5;
  uint32_t* tb = dyn;                           // [tbw] slots touched by this call
  int* hk = reinterpret_cast<int*>(dyn + tbw);  // [LRU_HT] page ids
  int* hv = hk + LRU_HT;                        // [LRU_HT] least index of the page
  int* slj = hv + LRU_HT;                       // [W] slot of a first occurrence
  int* mj = slj + LRU_LDS_W;                    // [W] misses' indices, first-occurrence order
  int* vic = mj + LRU_LDS_W;                    // [W] victim slots
  int* vold = vic + LRU_LDS_W;                  // [W] page each victim slot held
  int* mp = vold + LRU_LDS_W;                   // [W] misses' page ids

  // every state read up front
  const int par = c.hdr->parity;
  const int64_t clock_new = c.hdr->clock + 1;
  int pj[JPT], p2s[JPT];
#pragma unroll
  for (int u = 0; u < JPT; ++u) {
    const int j = tid + u * TKV_BLOCK;
    pj[u] = j < W ? needed[j] : -1;
  }
#pragma unroll
  for (int u = 0; u < JPT; ++u) p2s[u] = page_ok(c, pj[u]) ? c.page_to_slot[pj[u]] : -1;
  const int ch = (S + TKV_BLOCK - 1) / TKV_BLOCK;   // order entries per thread (<= LRU_CH)
  const int i0 = tid * ch;
  const int32_t* ord = c.order + (size_t)par * S;
  int sl[LRU_CH], sp[LRU_CH] = {};
#pragma unroll
  for (int u = 0; u < LRU_CH; ++u) sl[u] = (u < ch && i0 + u < S) ? ord[i0 + u] : 0;
#pragma unroll
  for (int u = 0; u < LRU_CH; ++u) {
    if (!(u < ch && i0 + u < S)) continue;
    if ((unsigned)sl[u] >= (unsigned)S) sl[u] = 0;   // never from a consistent state; keeps every access in bounds
    sp[u] = c.slot_to_page[sl[u]];
  }

  for (int w = tid; w < tbw; w += TKV_BLOCK) tb[w] = 0u;
  for (int h = tid; h < LRU_HT; h += TKV_BLOCK) {
    hk[h] = LRU_HT_EMPTY;
    hv[h] = 0x7FFFFFFF;
  }
  __syncthreads();

  // A: first occurrences (least index per valid page id)
  int hs[JPT];
  int bad = 0;
#pragma unroll
  for (int u = 0; u < JPT; ++u) {
    const int j = tid + u * TKV_BLOCK, p = pj[u];
    hs[u] = -1;
    if (j >= W || p == -1) continue;
    if (!page_ok(c, p)) { bad = 1; continue; }
    int h = lru_hash(p);
    while (true) {
      const int old = atomicCAS(&hk[h], LRU_HT_EMPTY, p);
      if (old == LRU_HT_EMPTY || old == p) break;
      h = (h + 1) & (LRU_HT - 1);
    }
    atomicMin(&hv[h], j);
    hs[u] = h;
  }
  if (bad) set_error(c.hdr, DERR_PAGE_RANGE);
  __syncthreads();
  bool first[JPT];
  int local = 0;
#pragma unroll
  for (int u = 0; u < JPT; ++u) {
    first[u] = hs[u] >= 0 && hv[hs[u]] == tid + u * TKV_BLOCK;
    local += first[u];
  }

  // B: the capacity check precedes any state change
  const int distinct = block_sum(local, sm_scan);
  if (distinct > S) {
#pragma unroll
    for (int u = 0; u < JPT; ++u) {
      const int j = tid + u * TKV_BLOCK;
      if (j < W && o.out_slots) o.out_slots[j] = -1;
    }
    if (tid == 0) {
      set_error(c.hdr, DERR_CAPACITY);
      *o.miss_count = 0;
    }
    return;
  }

  // C: hits are restamped; misses ranked in first-occurrence order (thread
  // t's entries are t and t + 256: rank the first half, then the second)
  int n_hits = 0, M = 0;
#pragma unroll
  for (int u = 0; u < JPT; ++u) {
    const int j = tid + u * TKV_BLOCK;
    int is_miss = 0;
    if (first[u]) {
      const int s = p2s[u];
      if (s >= 0) {
        touch_slot(tb, s);
        c.stamp[s] = clock_new;
        slj[j] = s;
        ++n_hits;
      } else {
        is_miss = 1;
      }
    }
    int tot;
    const int ex = block_excl_scan(is_miss, &tot, sm_scan);
    if (is_miss) {
      mj[M + ex] = j;
      mp[M + ex] = pj[u];
    }
    M += tot;
    if (u + 1 < JPT && (u + 1) * TKV_BLOCK >= W) break;
  }
  __syncthreads();

  // D: victims = the first M untouched entries of the (stamp, slot) order
  if (M > 0) {
    int cnt = 0;
    int cand[LRU_CH];
#pragma unroll
    for (int u = 0; u < LRU_CH; ++u) {
      cand[u] = (u < ch && i0 + u < S) && !slot_touched(tb, sl[u]);
      cnt += cand[u];
    }
    int tot;
    int r = block_excl_scan(cnt, &tot, sm_scan);
#pragma unroll
    for (int u = 0; u < LRU_CH; ++u)
      if (cand[u]) {
        if (r < M) {
          vic[r] = sl[u];
          vold[r] = sp[u];
        }
        ++r;
      }
    __syncthreads();
  }

  // E: bind each miss to its victim (an evicted page just loses its slot)
  int n_evict = 0;
  for (int m = tid; m < M; m += TKV_BLOCK) {
    const int j = mj[m], p = mp[m], s = vic[m], old = vold[m];
    if (old >= 0) {
      c.page_to_slot[old] = -1;
      ++n_evict;
    }
    c.page_to_slot[p] = s;
    c.slot_to_page[s] = p;
    c.stamp[s] = clock_new;
    touch_slot(tb, s);
    slj[j] = s;
  }
  __syncthreads();

  // fetch list: misses not marked no_fetch, in first-occurrence order
  int MF = 0;
  for (int base = 0; base < M; base += TKV_BLOCK) {
    const int m = base + tid;
    int f = 0, j = 0;
    if (m < M) {
      j = mj[m];
      f = (no_fetch && no_fetch[j]) ? 0 : 1;
    }
    int tot;
    const int ex = block_excl_scan(f, &tot, sm_scan);
    if (f) {
      o.miss[2 * (MF + ex)] = vic[m];
      o.miss[2 * (MF + ex) + 1] = mp[m];
    }
    MF += tot;
  }

  // F: out_slots (a duplicate reads its first occurrence's slot); fetch
  // flags (the page was not resident before this call and is fetched)
  if (o.out_slots) {
#pragma unroll
    for (int u = 0; u < JPT; ++u) {
      const int j = tid + u * TKV_BLOCK;
      if (j < W) o.out_slots[j] = hs[u] >= 0 ? slj[hv[hs[u]]] : -1;
    }
  }
  if (o.miss_flag) {
#pragma unroll
    for (int u = 0; u < JPT; ++u) {
      const int j = tid + u * TKV_BLOCK;
      if (j < W) o.miss_flag[j] = (hs[u] >= 0 && p2s[u] < 0 && !(no_fetch && no_fetch[hv[hs[u]]])) ? 1 : 0;
    }
  }

  // H: next order = untouched slots in old order, then touched slots by index
  {
    int32_t* nxt = c.order + (size_t)(1 - par) * S;
    int keep[LRU_CH], cnt = 0;
#pragma unroll
    for (int u = 0; u < LRU_CH; ++u) {
      keep[u] = (u < ch && i0 + u < S) && !slot_touched(tb, sl[u]);
      cnt += keep[u];
    }
    int tot;
    int r = block_excl_scan(cnt, &tot, sm_scan);
#pragma unroll
    for (int u = 0; u < LRU_CH; ++u)
      if (keep[u]) nxt[r++] = sl[u];
    const int run = tot;
    int t[LRU_CH];
    cnt = 0;
#pragma unroll
    for (int u = 0; u < LRU_CH; ++u) {
      t[u] = (u < ch && i0 + u < S) ? (int)slot_touched(tb, i0 + u) : 0;
      cnt += t[u];
    }
    r = run + block_excl_scan(cnt, &tot, sm_scan);
#pragma unroll
    for (int u = 0; u < LRU_CH; ++u)
      if (t[u]) nxt[r++] = i0 + u;
  }

  // I: clock, parity, counters
  const int hits = block_sum(n_hits, sm_scan);
  const int ev = block_sum(n_evict, sm_scan);
  if (tid == 0) {
    StateHdr* h = c.hdr;
    h->clock = clock_new;
    h->parity = 1 - par;
    h->counters[CNT_ENSURE] += 1;
    h->counters[CNT_HITS] += hits;
    h->counters[CNT_MISSES] += MF;
    h->counters[CNT_FRESH] += M - MF;
    h->counters[CNT_EVICT] += ev;
    *o.miss_count = MF;
  }
}

// A split store leaves the layer's blocks of the pages it began in a
// staging copy; a copy kernel moves them to the mirror rows later (beside
// the next attention).  A page this ensure has to fetch may be one of them
// -- written, evicted and needed again before that copy ran -- so its
// staged block is copied to its mirror row here, and the fetch that follows
// reads the row the pool held (the same bytes the later copy writes there).
// Misses are matched against the staged pages 256 at a time, the staged
// page list read through LDS in tiles.
__device__ void patch_staged_misses(const DevCtx& c, const EnsureOut& o) {
  constexpr int TILE = 1024;
  __shared__ int tile[TILE];
  __shared__ int hit[TKV_BLOCK];
  __syncthreads();                                         // the miss count and list are written
  const int m = *o.miss_count;
  const int L = c.stage_layer;
  bool patched = false;                                    // uniform
  for (int base = 0; base < m; base += TKV_BLOCK) {
    const int i = base + threadIdx.x;
    const int page = i < m ? o.miss[2 * i + 1] : -1;
    int found = -1;
    for (int t0 = 0; t0 < c.stage_n; t0 += TILE) {
      const int tn = min(TILE, c.stage_n - t0);
      __syncthreads();
      for (int u = threadIdx.x; u < tn; u += TKV_BLOCK) tile[u] = c.stage_page[t0 + u];
      __syncthreads();
      if (page >= 0 && found < 0)
        for (int u = 0; u < tn; ++u)
          if (tile[u] == page) {
            found = t0 + u;
            break;
          }
    }
    hit[threadIdx.x] = found;
    __syncthreads();
    const int nb = min(TKV_BLOCK, m - base);
    for (int k = 0; k < nb; ++k) {
      const int b = hit[k];                                // uniform
      if (b < 0) continue;
      patched = true;
      const int pg = o.miss[2 * (base + k) + 1];
      const uint4* src = reinterpret_cast<const uint4*>(c.stage + (size_t)b * c.layer_bytes);
      uint4* dst = reinterpret_cast<uint4*>(c.mirror + (size_t)pg * c.row_bytes + (size_t)L * c.layer_bytes);
      for (int64_t v = threadIdx.x; v < c.layer_bytes / 16; v += TKV_BLOCK) dst[v] = src[v];
    }
    __syncthreads();
  }
  if (patched) __threadfence_system();                     // the rows reach host memory before the fetch
}

// `dyn`: at least lru_lds_words(S) words of dynamic LDS.
__device__ void lru_ensure_block(const DevCtx& c, const int32_t* needed, int W,
                                 const uint8_t* no_fetch, EnsureOut o, int* sm_scan, uint32_t* dyn) {
  if (W <= LRU_LDS_W && lru_lds_fast_ok(c.S)) lru_ensure_lds(c, needed, W, no_fetch, o, sm_scan, dyn);
  else lru_ensure_global(c, needed, W, no_fetch, o, sm_scan, dyn);
  if (c.stage_layer >= 0) patch_staged_misses(c, o);
}
