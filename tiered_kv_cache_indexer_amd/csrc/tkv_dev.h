// Device-side definitions shared by the tiered KV-cache kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define TKV_BLOCK 256
#define TKV_WAVE 64
#define SEL_CHUNK 64   // pages scored per workgroup by the decode indexer scan

// device error word bits (mirror the TKV_ERR_* values of the public header)
#define DERR_PAGE_RANGE 1
#define DERR_CAPACITY 2
#define DERR_NOT_RESIDENT 4
#define DERR_BAD_MISS 8
#define DERR_RUN_LEN 16

enum { CNT_ENSURE = 0, CNT_HITS, CNT_MISSES, CNT_FRESH, CNT_EVICT, CNT_DROPS, CNT_BYTES_FETCHED,
       CNT_BYTES_MIRRORED, CNT_N };

struct StateHdr {
  int64_t clock;
  int64_t counters[CNT_N];
  int32_t error_word;
  int32_t parity;      // which half of `order` is current
  int32_t pad[2];
};

// Everything a kernel needs to find the tier's memory.  Passed by value.
struct DevCtx {
  int L, Hq, Hkv, D, PS, fp8;
  int64_t N;      // logical pages
  int S;          // slots
  int64_t row_bytes, layer_bytes, code_bytes;
  uint8_t* pool;
  uint8_t* mirror;          // device-visible address of the pinned host mirror
  uint16_t* slab;           // bf16 [L][N][Hkv][D]
  double* slab_acc;         // fp64 [L][N][Hkv][D] running key sums (exact for bf16 keys: see k_store)
  // residency state
  StateHdr* hdr;
  int32_t* page_to_slot;    // [N]
  int32_t* page_mark;       // [N], INT32_MAX when idle (first-occurrence scratch)
  int32_t* slot_to_page;    // [S]
  int64_t* stamp;           // [S]
  int32_t* order;           // [2][S] slots in ascending (stamp, slot)
  // workspace
  float* scores;            // [max_rows][max_pages rounded to 64] x 8 bytes: float scores or 64-bit keys
  int32_t* sel_slots;       // [max_rows][max_topk] slots of the selected pages (fused decode)
  uint16_t* qg;             // [max_rows][Hkv*D] per-group query sums (prefill scoring)
  int32_t* row_done;        // [max_rows] last-block counters (kept at zero between calls)
  int32_t* glob_done;       // [4]
  int32_t* slot_of_j;       // [max_width]
  int32_t* miss_j;          // [max_width]
  int32_t* victims;         // [max_width]
  int32_t* wneeded;         // [max_width]
  uint8_t* wnofetch;        // [max_width]
  int32_t* wmiss;           // [max_width][2]
  int32_t* wmiss_count;     // [1]
  float* attn_part;         // [max_batch][Hq][max_topk][D+2]
  int32_t* attn_done;       // [max_batch][Hkv]
  int32_t* iota;            // [max_rows + 1] = 0, 1, 2, ... (row_start of one-row-per-request calls)
  uint32_t* sel_bm;         // page bitmaps of requests with several rows, one per group of 64 of
                            // the request's rows: [max_rows/64 + max_batch][max_pages/32], kept at zero
  int32_t* pout;            // [max_width] preload ensure: slots
  int32_t* pmiss;           // [max_width][2] preload ensure: misses
  int32_t* pmiss_count;     // [1]
  float* attn_state;        // [max_rows][Hkv][ATTN_STATE_FLOATS] page-range attention records (or null)
  int32_t* bg_miss;         // [2][1 + 2*max_width] miss count and list kept for the split copy's later parts
  int32_t* rest_ctr;        // [2] work counter and finished waves of the rest-of-rows copy (zero between launches)
  uint8_t* miss_flag;       // [max_width] decode_layer: per needed entry, fetched by this call
  uint8_t* stage;           // [stage_blocks][layer_bytes] mirror blocks of the split store, copied later
  int32_t* stage_page;      // [stage_blocks] logical page of each staged block (-1: none)
  int stage_blocks;
  int stage_layer;          // layer of the staged blocks a split store's mirror copy may not have
                            // moved yet (-1: none); the ensure patches them into fetched rows
  int stage_n;              // staged blocks of that store
  int max_rows, max_pages, max_topk, max_batch, max_width;
  int attn_impl;            // ATTN_AUTO / ATTN_VECTOR / ATTN_MATRIX
  int attn_range_pages;     // pages per range of the multi-pass prefill attention (0 = one pass)
};

enum { ATTN_AUTO = 0, ATTN_VECTOR = 1, ATTN_MATRIX = 2 };
#define ATTN_STATE_FLOATS (8 * 32 * 4 + 8 * 2)
#define ATTN_RANGE_PAGES_DEFAULT 0

// Words of the selection bitmaps: sum over requests of ceil(rows_b / 64)
// groups is at most ceil(max_rows / 64) + max_batch.
inline size_t sel_bm_words(size_t max_rows, size_t max_batch, size_t max_pages) {
  return ((max_rows + 63) / 64 + max_batch) * ((max_pages + 31) / 32);
}

// ------------------------------------------------------------- call arguments --
struct SelArgs {
  int layer;
  const uint16_t* q;
  int rows;
  const int32_t* row_start;
  const int32_t* row_pos;
  const int32_t* bt;
  int max_pages;
  const int32_t* n_pages;
  int B;
  const float* bias;
  int topk;
  int32_t* sel_local;
  int32_t* needed;
  int C;
  int n_chunks;
  int do_ensure;
  int32_t* out_slots;
  int32_t* miss;
  int32_t* miss_count;
  int32_t* sel_slots;   // fused path: translated slots of sel_local (or null)
  uint8_t* miss_flag;   // fused path: per needed entry, 1 where this call fetches its page (or null)
  int one_row_each;     // 1: row r is request r's only row (row_start = 0, 1, ..., B)
};

struct StoreArgs {
  uint8_t* stage;        // split store: mirror blocks of pages the write begins go here (null: direct)
  int32_t* stage_page;
  int stage_blocks;
  int layer;
  const uint16_t* k;
  const uint16_t* v;
  int n_runs;
  const int32_t* run_req;
  const int32_t* run_start;
  const int32_t* run_len;
  const int32_t* run_tok_off;
  const int32_t* bt;
  int max_pages;
};

struct AttnArgs {
  int layer;
  const uint16_t* q;
  int rows;
  const int32_t* row_start;
  const int32_t* row_pos;
  const int32_t* ctx_len;
  const int32_t* sel;
  const int32_t* bt;
  int max_pages;
  int topk;
  int B;
  uint16_t* out;
  const int32_t* slots;  // optional: slots of sel (skips the page->slot translation)
  int slots_stride;      // row stride of `slots` (0: topk)
  int one_row_each;      // 1: row r is request r's only row (row_start = 0, 1, ..., B)
  int host_tail;         // read pages that are not resident from their mirror row
  // Fetch folded into the launch (decode_layer, split mode): extra
  // workgroups copy the rows of the miss list (fmiss, *fmiss_count pairs of
  // slot and page, at most fwidth) for every layer but this one; an entry
  // whose slot_miss flag is set (same indexing as `slots`) is read from the
  // mirror row of page slot_page[...] and its block of this layer is written
  // to the slot by the wave that folds it.
  const int32_t* fmiss;
  const int32_t* fmiss_count;
  int fwidth;
  const uint8_t* slot_miss;
  const int32_t* slot_page;
  int splits;
  int pages_per_split;
};

// ------------------------------------------------------------------ numbers --
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// binary32 -> bfloat16, round to nearest, ties to even
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// binary32 -> OCP E4M3FN, round to nearest, ties to even, saturating to +-448.
// Normal results: the IEEE exponent/mantissa field rounded to 3 mantissa bits
// and rebiased (127 -> 7); subnormal results: round(|x| * 2^9) to an integer.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;   // >= 448 (and inf): saturate
  if (a >= 0x3C800000u) {                      // >= 2^-6: normal
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));
  }
  float m = rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE to integer 0..8
  return sign | (uint32_t)m;
}

// e4m3 byte pair decode through the hardware converter (gfx950: OCP E4M3FN)
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 e4m3x2_lo(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false); }
__device__ __forceinline__ f32x2 e4m3x2_hi(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true); }

// orderable key: larger float -> larger unsigned (+0 canonical)
__device__ __forceinline__ uint32_t f32_order(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------ wave sorting --
// 64-bit selection keys: (orderable score << 32) | ~index -- a larger key is a
// higher score, and among equal scores the lower index.  0 = no page.
__device__ __forceinline__ uint64_t sel_key(float score, int idx) {
  return ((uint64_t)f32_order(score) << 32) | (uint64_t)(~(uint32_t)idx);
}
__device__ __forceinline__ int sel_key_index(uint64_t k) { return (int)(~(uint32_t)k); }

// The value of lane (lane ^ m) for the constant distances of the wave sort
// networks (m folds to a constant once the networks are unrolled): DPP moves
// for 1, 2 (quad permutes) and 8 (row rotate by 8), a ds_swizzle in bit-mask
// mode for 4 and 16 (within 32 lanes), a lane permute for 32.
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v, int m) {
  switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
    case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
    default: return (uint32_t)__shfl_xor((int)v, m, 64);
  }
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = xor_lane_u32((uint32_t)v, m), hi = xor_lane_u32((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double xor_lane_f64(double v, int m) {
  return __longlong_as_double((long long)shfl_xor_u64((uint64_t)__double_as_longlong(v), m));
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((int)(uint32_t)v, src, 64), hi = __shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one key per lane across a wave, descending (lane 0 = max).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = shfl_xor_u64(v, stride);
      const bool lower = (lane & stride) == 0;
      const bool desc = (lane & size) == 0;
      const bool keep_max = (lower == desc);
      v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  return v;
}

// Top 64 of two descending lists, descending.
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t a, uint64_t b) {
  const int lane = threadIdx.x & 63;
  const uint64_t br = shfl_u64(b, 63 - lane);
  uint64_t v = a > br ? a : br;   // bitonic, holds the top 64
#pragma unroll
  for (int stride = 32; stride > 0; stride >>= 1) {
    const uint64_t o = shfl_xor_u64(v, stride);
    const bool lower = (lane & stride) == 0;
    v = lower ? (v > o ? v : o) : (v < o ? v : o);
  }
  return v;
}

// Bitonic sort of one int per lane, ascending.
__device__ __forceinline__ int wave_sort_asc_i32(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int o = (int)xor_lane_u32((uint32_t)v, stride);
      const bool lower = (lane & stride) == 0;
      const bool asc = (lane & size) == 0;
      const bool keep_min = (lower == asc);
      v = keep_min ? min(v, o) : max(v, o);
    }
  }
  return v;
}

// ------------------------------------------------------------------ block ops --
// Inclusive prefix sum across the wave by DPP: row shifts right by 1, 2, 4
// and 8 (a lane whose source lies outside its 16-lane row adds 0), then lane
// 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Sum / max over the wave, every lane gets the result (xor butterflies).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __uint_as_float(xor_lane_u32(__float_as_uint(v), o));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __uint_as_float(xor_lane_u32(__float_as_uint(v), o)));
  return v;
}

// Block-wide exclusive scan of one int per thread (blockDim == 256).
// Returns the exclusive prefix; *total gets the block sum.  Uses sm[0..4].
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* sm) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) sm[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < TKV_BLOCK / 64; ++i) {
    int s = sm[i];
    if (i < w) base += s;
    tot += s;
  }
  *total = tot;
  return base + inc - v;
}

__device__ __forceinline__ int block_sum(int v, int* sm) {
  int tot;
  (void)block_excl_scan(v, &tot, sm);
  return tot;
}

__device__ __forceinline__ int ld_acquire_i32(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void set_error(StateHdr* h, int bits) {
  atomicOr(&h->error_word, bits);
}

// Last-block election: every block calls it once after publishing its
// results; returns true in exactly one block (the last to arrive), after
// which that block sees every other block's writes.  The counter is reset.
// Each wave first drains its own memory operations (so its stores have
// reached L2), then one thread per block makes the block's writes visible
// device-wide (agent-scope release: L2 writeback) before counting in, and the
// last block's thread 0 acquires (L1/L2 invalidate) for the whole block --
// one fence per block instead of one per thread.
__device__ __forceinline__ bool last_block_arrive(int32_t* counter, int expected, int* sm_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == expected - 1);
    if (last) {
      __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    *sm_flag = last;
  }
  __syncthreads();
  return *sm_flag != 0;
}
