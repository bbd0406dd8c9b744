// store_kv with the write-through mirror (gfx950).
//
// FreeToken PR #499, "Design": each store is also written to the pinned host
// mirror through the device-visible mapping, so a slot never holds bytes the
// mirror lacks and evicting it costs nothing.  PR #525 commit summary
// (mirror_store_quant): the mirror gets the quantiser's output, the e4m3
// codes and fp32 scales the pool gets, not the values from before it.
//
// One workgroup per (run, page of the run).  A wave takes groups of four page
// positions, loads the group's K and V rows at once and quantises one token
// at a time: each lane holds 8 of the token's Hkv*d bf16 values (one 16-byte
// load), the wave reduces |x| to the token's amax, scale = amax/448 (1 if
// amax is 0), code = e4m3(x / scale) with a correctly rounded fp32 division.
// K codes go straight to the pool slot (HBM) and the mirror row (posted
// writes over the host link), 8 bytes per lane.  V codes are stored
// transposed ([h][d][page]): each lane packs its 8 rows' bytes for 4
// consecutive positions into words, the block is staged in LDS and written
// out row by row.  The workgroup also sums the page's keys for the indexer
// slab: slab = bf16(fp32(running sum) / tokens written).  The sums are fp64:
// every bf16 key of a page feature is a multiple of 2^e (e the lowest set
// bit among them) and every partial sum is bounded by sum |key|, so while
// sum |key| < 2^(53+e) -- any page of normally distributed bf16 keys -- each
// fp64 addition is exact and the result does not depend on the order the
// waves add in; fp32 sums would round once the keys span more than 24 bits.
#include "tkv_dev.h"
#include "tkv_launch.h"

// 16 waves: one group of four positions each on a 64-token page, so the
// quantisation of a page is done in a quarter of the time it took 4 waves
// and the mirror writes that follow start sooner (the writes run at the
// link's rate; measured on MI355X, a 4,096-token store of 12 layers took
// 1.5 ms, 0.7 ms of it with the host writes taken out)
// (Hkv*d = 1024 keeps 4 waves: its registers would not fit 16)
template <int E8>
__host__ __device__ constexpr int store_block() { return E8 >= 128 ? 256 : 1024; }



template <int E8, bool FP8>
__global__ __launch_bounds__(store_block<E8>()) void k_store(DevCtx c, StoreArgs a) {
  constexpr int E = E8 * 8;
  constexpr int SPL = E8 >= 64 ? E8 / 64 : 1;
  constexpr int VT_WORDS = FP8 ? E * (64 / 4 + 1) : 1;   // transposed V block, rows padded by one word
  // fp8 K codes and both scale vectors staged too (up to Hkv*d = 512), so
  // every byte leaves in 16-byte vectors, a wave's store one contiguous KiB
  constexpr bool STAGE_K = FP8 && E8 <= 64;
  constexpr int STORE_BLOCK = store_block<E8>();
  constexpr int NW = STORE_BLOCK / 64;
  __shared__ double ksum_w[NW][E];
  __shared__ uint32_t vt[VT_WORDS];
  __shared__ __align__(16) uint8_t kt[STAGE_K ? E * 64 : 16];
  __shared__ __align__(16) float sct[STAGE_K ? 2 * 64 : 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x, j = blockIdx.y;
  const int PS = c.PS, D = c.D;
  const int blk = r * (int)gridDim.y + j;                  // staging block of the split store
  if (a.stage && tid == 0 && blk < a.stage_blocks) a.stage_page[blk] = -1;
  const int req = a.run_req[r], start = a.run_start[r], len = a.run_len[r];
  if (len <= 0) return;
  // the grid reaches gridDim.y pages of the run: a longer run is flagged
  if (j == 0 && tid == 0 && (start + len - 1) / PS - start / PS >= (int)gridDim.y) set_error(c.hdr, DERR_RUN_LEN);
  const int lp = start / PS + j;
  const int t0 = max(start, lp * PS), t1 = min(start + len, (lp + 1) * PS);
  if (t0 >= t1) return;
  if (lp >= a.max_pages) {
    if (tid == 0) set_error(c.hdr, DERR_PAGE_RANGE);
    return;
  }
  const int off = t0 - lp * PS, n = t1 - t0;
  const int page = a.bt[(size_t)req * a.max_pages + lp];
  if (page < 0 || (int64_t)page >= c.N) {
    if (tid == 0) set_error(c.hdr, DERR_PAGE_RANGE);
    return;
  }
  const int slot = c.page_to_slot[page];
  if (slot < 0 && tid == 0) set_error(c.hdr, DERR_NOT_RESIDENT);
  // split store: a write that begins the page defines the page's whole block
  // of this layer (written positions, zero-filled tail), so it is built in
  // the staging copy and moved to the mirror afterwards; other writes go to
  // the mirror directly
  const bool staged = a.stage && off == 0 && blk < a.stage_blocks;
  uint8_t* mir = staged ? a.stage + (size_t)blk * c.layer_bytes
                        : c.mirror + (size_t)page * c.row_bytes + (size_t)a.layer * c.layer_bytes;
  if (staged && tid == 0) a.stage_page[blk] = page;
  uint8_t* pol = slot >= 0 ? c.pool + (size_t)slot * c.row_bytes + (size_t)a.layer * c.layer_bytes : nullptr;
  const size_t cb = (size_t)c.code_bytes;
  const int tok_first = a.run_tok_off[r] + (t0 - start);  // input row of page position `off`
  const int VROW = PS / 4 + 1;                             // words per staged V row (fp8)
  if (FP8)
    for (int w = tid; w < E * VROW; w += STORE_BLOCK) vt[w] = 0u;

  double ksum[SPL][8];
#pragma unroll
  for (int s = 0; s < SPL; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) ksum[s][t] = 0.0;
  if (FP8) __syncthreads();

  // a wave handles groups of 4 consecutive page positions
  for (int grp = wave; grp * 4 < PS; grp += NW) {
    const int pbase = grp * 4;
    if (pbase + 3 < off || pbase >= off + n) continue;   // wave-uniform
    uint32_t vpack[SPL][8];
#pragma unroll
    for (int s = 0; s < SPL; ++s)
#pragma unroll
      for (int t = 0; t < 8; ++t) vpack[s][t] = 0u;
    // the group's K and V rows (4 positions) in flight together: one load
    // latency per group instead of one per token and tensor
    uint4 rawg[4][2][SPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pos = pbase + u;
      const bool in = pos >= off && pos < off + n;
      const int tok = tok_first + (pos - off);
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        const uint16_t* src = (kv == 0 ? a.k : a.v) + (size_t)(in ? tok : 0) * E;
#pragma unroll
        for (int s = 0; s < SPL; ++s) {
          const int seg = lane + s * 64;
          rawg[u][kv][s] = (in && seg < E8) ? reinterpret_cast<const uint4*>(src)[seg] : make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pos = pbase + u;
      if (pos < off || pos >= off + n) continue;         // wave-uniform
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        float x[SPL][8];
        bool act[SPL];
        uint4 raw[SPL];
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < SPL; ++s) {
          const int seg = lane + s * 64;
          act[s] = seg < E8;
          raw[s] = rawg[u][kv][s];
          const uint32_t ww[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            x[s][2 * t] = __uint_as_float(ww[t] << 16);
            x[s][2 * t + 1] = __uint_as_float(ww[t] & 0xFFFF0000u);
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) amax = fmaxf(amax, fabsf(x[s][t]));
          if (kv == 0)
#pragma unroll
            for (int t = 0; t < 8; ++t) ksum[s][t] += (double)x[s][t];
        }
        uint8_t* mblk = mir + kv * cb;
        uint8_t* pblk = pol ? pol + kv * cb : nullptr;
        if (FP8) {
          amax = wave_max(amax);
          const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
          for (int s = 0; s < SPL; ++s) {
            if (!act[s]) continue;
            uint32_t code[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) code[t] = f32_to_e4m3(x[s][t] / scale);
            if (kv == 0) {
              // K codes [h][pos][d]: 8 consecutive bytes
              const int e = (lane + s * 64) * 8, h = e / D, dd = e - h * D;
              const uint2 val = make_uint2(code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24,
                                           code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24);
              const size_t o = ((size_t)h * PS + pos) * D + dd;
              if (STAGE_K) {
                *reinterpret_cast<uint2*>(kt + o) = val;
              } else {
                *reinterpret_cast<uint2*>(mblk + o) = val;
                if (pblk) *reinterpret_cast<uint2*>(pblk + o) = val;
              }
            } else {
              // V codes transposed [h][d][pos]: byte u of the group's word in each of 8 rows
#pragma unroll
              for (int t = 0; t < 8; ++t) vpack[s][t] |= code[t] << (8 * u);
            }
          }
          if (lane == 0) {
            if (STAGE_K) {
              sct[kv * 64 + pos] = scale;
            } else {
              const size_t so = 2 * cb + (size_t)kv * PS * 4 + (size_t)pos * 4;
              *reinterpret_cast<float*>(mir + so) = scale;
              if (pol) *reinterpret_cast<float*>(pol + so) = scale;
            }
          }
        } else {
#pragma unroll
          for (int s = 0; s < SPL; ++s) {
            if (!act[s]) continue;
            const int e = (lane + s * 64) * 8, h = e / D, dd = e - h * D;
            const size_t o = (((size_t)h * PS + pos) * D + dd) * 2;
            *reinterpret_cast<uint4*>(mblk + o) = raw[s];
            if (pblk) *reinterpret_cast<uint4*>(pblk + o) = raw[s];
          }
        }
      }
    }
    if (FP8) {
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        if (lane + s * 64 >= E8) continue;
#pragma unroll
        for (int t = 0; t < 8; ++t) vt[((lane + s * 64) * 8 + t) * VROW + grp] = vpack[s][t];
      }
    }
  }

  // a write that begins the page clears the page's later positions
  const bool zero_tail = (off == 0 && n < PS);
  if (zero_tail) {
    const int elt = FP8 ? 1 : 2;
    const int H = c.Hkv;
    const int tail = (PS - n) * D * elt;  // K bytes per head (and V bytes for bf16)
    for (int kv = 0; kv < (FP8 ? 1 : 2); ++kv)
      for (int h = 0; h < H; ++h) {
        const size_t base = (size_t)kv * cb + ((size_t)h * PS + n) * D * elt;
        for (int i = tid * 4; i < tail; i += STORE_BLOCK * 4) {
          *reinterpret_cast<uint32_t*>(mir + base + i) = 0u;
          if (pol) *reinterpret_cast<uint32_t*>(pol + base + i) = 0u;
        }
      }
    if (FP8) {
      for (int i = n + tid; i < PS; i += STORE_BLOCK) {
        reinterpret_cast<float*>(mir + 2 * cb)[i] = 0.f;
        reinterpret_cast<float*>(mir + 2 * cb + PS * 4)[i] = 0.f;
        if (pol) {
          reinterpret_cast<float*>(pol + 2 * cb)[i] = 0.f;
          reinterpret_cast<float*>(pol + 2 * cb + PS * 4)[i] = 0.f;
        }
      }
    }
  }

  if (FP8) {
    // transposed V rows out: positions [off, off+n) (through the page end when it begins the page)
    __syncthreads();
    const int lo = off, hi = zero_tail ? PS : off + n;
    uint8_t* mv = mir + cb;
    uint8_t* pv = pol ? pol + cb : nullptr;
    const int wpr = PS / 4;
    if (STAGE_K) {
      // K codes [h][pos][d]: positions [off, off+n) of each head, 16 bytes a thread
      const int per_h = n * D / 16;
      for (int g16 = tid; g16 < c.Hkv * per_h; g16 += STORE_BLOCK) {
        const int h = g16 / per_h;
        const size_t o = ((size_t)h * PS + off) * D + (size_t)(g16 - h * per_h) * 16;
        const uint4 w = *reinterpret_cast<const uint4*>(kt + o);
        *reinterpret_cast<uint4*>(mir + o) = w;
        if (pol) *reinterpret_cast<uint4*>(pol + o) = w;
      }
      // scales of positions [off, off+n), K then V
      for (int i = tid; i < 2 * n; i += STORE_BLOCK) {
        const int kv = i / n, pos = off + (i - kv * n);
        const size_t so = 2 * cb + (size_t)kv * PS * 4 + (size_t)pos * 4;
        const float sc = sct[kv * 64 + pos];
        *reinterpret_cast<float*>(mir + so) = sc;
        if (pol) *reinterpret_cast<float*>(pol + so) = sc;
      }
    }
    if (STAGE_K && lo == 0 && hi == PS) {
      // whole V rows: 16 bytes (four staged words) a thread, rows back to back
      const int gpr = PS / 16;
      for (int g16 = tid; g16 < E * gpr; g16 += STORE_BLOCK) {
        const int e = g16 / gpr, part = g16 - e * gpr;
        const uint32_t* src = vt + e * VROW + part * 4;
        const uint4 w = make_uint4(src[0], src[1], src[2], src[3]);
        const size_t o = (size_t)e * PS + part * 16;
        *reinterpret_cast<uint4*>(mv + o) = w;
        if (pv) *reinterpret_cast<uint4*>(pv + o) = w;
      }
    } else {
    for (int idx = tid; idx < E * wpr; idx += STORE_BLOCK) {
      const int e = idx / wpr, w = idx - e * wpr;
      const int p0 = 4 * w;
      if (p0 + 4 <= lo || p0 >= hi) continue;
      const uint32_t word = vt[e * VROW + w];
      const size_t o = (size_t)e * PS + p0;
      if (p0 >= lo && p0 + 4 <= hi) {
        *reinterpret_cast<uint32_t*>(mv + o) = word;
        if (pv) *reinterpret_cast<uint32_t*>(pv + o) = word;
      } else {
        for (int b = 0; b < 4; ++b) {
          if (p0 + b < lo || p0 + b >= hi) continue;
          mv[o + b] = (uint8_t)(word >> (8 * b));
          if (pv) pv[o + b] = (uint8_t)(word >> (8 * b));
        }
      }
    }
    }
  }

  // slab: mean of every key written to this page so far
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int seg = lane + s * 64;
    if (seg < E8)
#pragma unroll
      for (int t = 0; t < 8; ++t) ksum_w[wave][seg * 8 + t] = ksum[s][t];
  }
  __syncthreads();
  const size_t sbase = ((size_t)a.layer * c.N + page) * E;
  const int cnt = off + n;
  for (int e = tid; e < E; e += STORE_BLOCK) {
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < NW; w += 4) sum += (ksum_w[w][e] + ksum_w[w + 1][e]) + (ksum_w[w + 2][e] + ksum_w[w + 3][e]);
    if (off > 0) sum += c.slab_acc[sbase + e];
    c.slab_acc[sbase + e] = sum;
    c.slab[sbase + e] = f32_to_bf16((float)sum / (float)cnt);
  }
  if (tid == 0) {
    const int64_t tok_bytes = c.layer_bytes / PS;
    const int64_t nb = (int64_t)(n + (off == 0 ? PS - n : 0)) * tok_bytes;
    atomicAdd((unsigned long long*)&c.hdr->counters[CNT_BYTES_MIRRORED], (unsigned long long)nb);
  }
}

// The split store's second half: each staged block (one per store
// workgroup) to its page's mirror row, this layer's block.  A small grid
// walks (block, 16 KiB part) items with four 16-byte vectors in flight per
// thread: like the rest-of-rows copy's host reads, host writes from a grid
// spread over every CU slow the kernels running beside them (the selection
// of a 4,096-row chunk took 0.13 ms a layer instead of 0.06 with 260
// workgroups writing).  The library enqueues it beside the layer's
// attention, which it slows by about 2% (8.95 -> 9.1-9.2 ms a 4,096-token
// chunk), where beside the selection 16 workgroups still doubled that.
#ifndef MIRROR_COPY_GRID
#define MIRROR_COPY_GRID 16
#endif
__global__ __launch_bounds__(TKV_BLOCK) void k_mirror_copy(DevCtx c, int layer, int blocks) {
  constexpr int PART = 16384 / 16;            // vectors per item
  const int64_t nvec = c.layer_bytes / 16;
  const int parts = (int)((nvec + PART - 1) / PART);
  const int items = blocks * parts;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int b = it / parts, part = it - b * parts;
    const int page = c.stage_page[b];
    if (page < 0 || (int64_t)page >= c.N) continue;
    const uint4* src = reinterpret_cast<const uint4*>(c.stage + (size_t)b * c.layer_bytes);
    uint4* dst = reinterpret_cast<uint4*>(c.mirror + (size_t)page * c.row_bytes + (size_t)layer * c.layer_bytes);
    const int64_t v0 = (int64_t)part * PART, v1 = min(nvec, v0 + PART);
    for (int64_t v = v0 + threadIdx.x; v < v1; v += 4 * TKV_BLOCK) {
      uint4 t[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (v + u * TKV_BLOCK < v1) t[u] = src[v + u * TKV_BLOCK];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (v + u * TKV_BLOCK < v1) dst[v + u * TKV_BLOCK] = t[u];
    }
  }
}

hipError_t launch_mirror_copy(const DevCtx& c, int layer, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(k_mirror_copy, dim3(MIRROR_COPY_GRID), dim3(TKV_BLOCK), 0, st, c, layer, blocks);
  return hipGetLastError();
}

hipError_t launch_store(const DevCtx& c, const StoreArgs& a, int max_run_len, hipStream_t st) {
  const int ppr = (max_run_len + c.PS - 1) / c.PS + 1;
  dim3 grid(a.n_runs, ppr);
  const int E8 = c.Hkv * c.D / 8;
  if (c.fp8) {
    if (E8 == 64) hipLaunchKernelGGL((k_store<64, true>), grid, dim3(store_block<64>()), 0, st, c, a);
    else if (E8 == 16) hipLaunchKernelGGL((k_store<16, true>), grid, dim3(store_block<16>()), 0, st, c, a);
    else if (E8 == 32) hipLaunchKernelGGL((k_store<32, true>), grid, dim3(store_block<32>()), 0, st, c, a);
    else if (E8 == 128) hipLaunchKernelGGL((k_store<128, true>), grid, dim3(store_block<128>()), 0, st, c, a);
    else return hipErrorInvalidValue;
  } else {
    if (E8 == 64) hipLaunchKernelGGL((k_store<64, false>), grid, dim3(store_block<64>()), 0, st, c, a);
    else if (E8 == 16) hipLaunchKernelGGL((k_store<16, false>), grid, dim3(store_block<16>()), 0, st, c, a);
    else if (E8 == 32) hipLaunchKernelGGL((k_store<32, false>), grid, dim3(store_block<32>()), 0, st, c, a);
    else if (E8 == 128) hipLaunchKernelGGL((k_store<128, false>), grid, dim3(store_block<128>()), 0, st, c, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
