// Sparse paged attention on the matrix cores (gfx950): fp8 e4m3 KV with
// per-token scales, 64-token pages, d = 128, 8 query heads per KV head.
//
// FreeToken PR #499, "Design": after the ensure, attention reads only the
// selected pages through the logical->physical translation; vLLM RFC #33980,
// "Proposed Change": attention over the top-k KV.  The arithmetic is the
// same softmax as the vector kernel; the products move to the matrix cores:
// S = Q.K^T on the fp8 instruction v_mfma_scale_f32_16x16x128_f8f6f4 (K codes
// as stored; the query scaled by a power of two and split into two e4m3
// parts, exact for bf16 queries with up to 8 significant bits), and P.V on
// v_mfma_f32_16x16x32_bf16 (e4m3 V codes are exact in bf16).
//
// One wave processes one selected page of one (row, KV head) at a time.
//  * S^T = K . Q^T: the 64 keys of the page are four 16-row A tiles, the
//    8 query heads are B columns 0..7 (columns 8..15 zero).  The
//    contraction over d runs in an order in which a lane's A slice is two
//    16-byte loads of its key row (32 fp8 codes); the query operand (built
//    once per (row, KV head)) uses the same order.  Row m of A tile `mt` is token 16*(m/4) + 4*mt + m%4, so
//    the output fragment of lane (q = lane/16, h = lane%16) holds tokens
//    16q .. 16q+15 of head h: the online softmax is per lane plus two
//    cross-lane reductions.
//  * The probabilities, times the token's V scale and rounded to bf16, are
//    then already the B operand of O^T += V^T . P^T: lane (q, h) supplies
//    tokens 16q + 8*kt .. +7 of head h for contraction step kt.  fp8 V is
//    stored transposed ([d][page]), so the matching A slice (one d row,
//    16 tokens) is one 16-byte load.  The accumulator columns are the
//    heads, so the softmax rescale is one multiply per lane.
// Wave-per-row mode (many rows, e.g. prefill chunks): each wave owns one
// (row, KV head) and runs over all its pages; nothing is merged.  Split
// mode (decode): a workgroup of 4 waves owns a (row, KV head, page range),
// the waves' states are merged in LDS, and split records are merged by the
// last workgroup to arrive.
#include "tkv_dev.h"
#include "tkv_launch.h"
#include "tkv_attn_dev.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int MD = ATT_D, MG = ATT_G, MPS = 64, MWAVES = TKV_BLOCK / 64;

__device__ __forceinline__ uint32_t bits2(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Page rows are pool slots or mapped mirror rows, both global memory; the
// row pointer is rebuilt from lane values, so say so explicitly (otherwise
// the loads become flat loads).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ T gld(const uint8_t* p) {
  static_assert(sizeof(T) == 16, "16-byte loads");
  const u32x4v v = *(const __attribute__((address_space(1))) u32x4v*)(p);
  return __builtin_bit_cast(T, v);
}

// 16 e4m3 codes (bytes in address order) -> bf16 operands of elements 0..7
// and 8..15 (exact conversion)
__device__ __forceinline__ void fp8x16_to_bf16(const uint4 w, bf16x8& lo, bf16x8& hi) {
  const uint4 l = make_uint4(bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.0f, false)),
                             bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.0f, true)),
                             bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.0f, false)),
                             bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.0f, true)));
  const uint4 h = make_uint4(bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.z, 1.0f, false)),
                             bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.z, 1.0f, true)),
                             bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.w, 1.0f, false)),
                             bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.w, 1.0f, true)));
  lo = __builtin_bit_cast(bf16x8, l);
  hi = __builtin_bit_cast(bf16x8, h);
}

__device__ __forceinline__ bf16x8 ld_q8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

struct WaveAttn {
  f32x4 acc[8];   // O^T tiles: d = 16*dt + 4*(lane/16) + v, head lane%16
  float m_run, l_run;
};

// Query operand of S^T = K.Q^T on the fp8 matrix cores
// (v_mfma_scale_f32_16x16x128_f8f6f4: lane l supplies row l%16 of A and
// column l%16 of B over contraction indices 32*(l/16) .. +31, one byte each).
// The K codes are the A operand as stored.  The query, scaled by 2^-e so its
// largest magnitude is in [128, 256), is split into two e4m3 parts,
// q' = hi + lo (hi = e4m3(q'), lo = e4m3(q' - hi)); the instruction's E8M0
// B scale 2^e undoes the scaling exactly.  For a query on a 2^-5 grid
// bounded by 4 the split is exact; in general hi + lo carries 8 significant
// bits, as the bf16 query does.
struct QOp {
  i32x8 hi, lo;
  int scale;   // E8M0: 127 + e
};

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c2, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, d, w, true);
  return (uint32_t)w;
}

// The row's query slice this lane needs: head lane%16 (< 8), elements
// 32*(lane/16) .. +31, as raw bf16 (four 16-byte loads).
__device__ __forceinline__ void load_query_raw(const AttnArgs& a, const DevCtx& c, int r, int g, int lane,
                                               uint4 (&raw)[4]) {
  const int h = lane & 15, q = lane >> 4;
  if (h < MG) {
    const uint16_t* qh = a.q + ((size_t)r * c.Hq + g * MG + h) * MD + 32 * q;
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[u] = *reinterpret_cast<const uint4*>(qh + 8 * u);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[u] = make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void make_qop(const uint4 (&raw)[4], QOp& qo) {
  float x[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t ww[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      x[8 * u + 2 * t] = __uint_as_float(ww[t] << 16);
      x[8 * u + 2 * t + 1] = __uint_as_float(ww[t] & 0xFFFF0000u);
    }
  }
  // the wave's largest magnitude -> e with max * 2^-e in [128, 256)
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(x[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  int e = 0;
  if (mx > 0.f) e = min(max(ilogbf(mx) - 7, -126), 126);
  qo.scale = 127 + e;
  uint32_t hw[8], lw[8];
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    float y[4], lo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) y[t] = ldexpf(x[i + t], -e);
    const uint32_t hb = fp8x4(y[0], y[1], y[2], y[3]);
    const f32x2 h01 = e4m3x2_lo(hb), h23 = e4m3x2_hi(hb);
    lo[0] = y[0] - h01.x; lo[1] = y[1] - h01.y; lo[2] = y[2] - h23.x; lo[3] = y[3] - h23.y;
    hw[i / 4] = hb;
    lw[i / 4] = fp8x4(lo[0], lo[1], lo[2], lo[3]);
  }
  qo.hi = i32x8{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
  qo.lo = i32x8{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
}

__device__ __forceinline__ void load_query(const AttnArgs& a, const DevCtx& c, int r, int g, int lane, QOp& qo) {
  uint4 raw[4];
  load_query_raw(a, c, r, g, lane, raw);
  make_qop(raw, qo);
}

// One page of one KV head in registers: K codes as the fp8 A operand of the
// four S tiles, V^T codes (16 tokens of one d row per lane and d tile), and
// the K and V scales of the 16 tokens this lane's output fragment holds.
struct PageRegs {
  i32x8 ka[4];
  uint4 vr[8];
  float4 ks4[4], vs4[4];   // K / V scales of tokens 16q + 4i .. +3 (q = lane / 16)
};

__device__ __forceinline__ void load_page(const uint8_t* blk, size_t cb, int g, int lane, PageRegs& pr) {
  const int m = lane & 15, q = lane >> 4;
  const uint8_t* kb = blk + (size_t)g * MPS * MD;
  const uint8_t* vb = blk + cb + (size_t)g * MPS * MD;
  const uint8_t* sc = blk + 2 * cb;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int t = 16 * (m >> 2) + 4 * mt + (m & 3);
    const uint4 k0 = gld<uint4>(kb + t * MD + 32 * q);
    const uint4 k1 = gld<uint4>(kb + t * MD + 32 * q + 16);
    pr.ka[mt] = i32x8{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) pr.vr[dt] = gld<uint4>(vb + (16 * dt + m) * MPS + 16 * q);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr.ks4[i] = gld<float4>(sc + 4 * (16 * q + 4 * i));
    pr.vs4[i] = gld<float4>(sc + 4 * MPS + 4 * (16 * q + 4 * i));
  }
}

// The block `load_page` read, written to `blk` (a pool slot's block of this
// layer): every lane stores what it loaded; the scales (one pair per token,
// shared by the KV heads) from head 0's wave, one lane per 16.
__device__ __forceinline__ void store_page(uint8_t* blk, size_t cb, int g, int lane, const PageRegs& pr) {
  const int m = lane & 15, q = lane >> 4;
  uint8_t* kb = blk + (size_t)g * MPS * MD;
  uint8_t* vb = blk + cb + (size_t)g * MPS * MD;
  uint8_t* sc = blk + 2 * cb;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int t = 16 * (m >> 2) + 4 * mt + (m & 3);
    const i32x8 k = pr.ka[mt];
    *reinterpret_cast<uint4*>(kb + t * MD + 32 * q) = make_uint4((uint32_t)k[0], (uint32_t)k[1], (uint32_t)k[2], (uint32_t)k[3]);
    *reinterpret_cast<uint4*>(kb + t * MD + 32 * q + 16) =
        make_uint4((uint32_t)k[4], (uint32_t)k[5], (uint32_t)k[6], (uint32_t)k[7]);
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<uint4*>(vb + (16 * dt + m) * MPS + 16 * q) = pr.vr[dt];
  if (g == 0 && m == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<float4*>(sc + 4 * (16 * q + 4 * i)) = pr.ks4[i];
      *reinterpret_cast<float4*>(sc + 4 * MPS + 4 * (16 * q + 4 * i)) = pr.vs4[i];
    }
  }
}

// Fold one loaded page (nt >= 1 visible tokens) into the wave's running state.
__device__ __forceinline__ void fold_page(const PageRegs& pr, int nt, int lane, const QOp& qo, float qscale,
                                          WaveAttn& st) {
  const int q = lane >> 4;
  // S^T tiles: two fp8 products per 16 keys (query hi and lo parts)
  f32x4 s[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pr.ka[mt], qo.hi, z, 0, 0, 0, 127, 0, qo.scale);
    z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pr.ka[mt], qo.lo, z, 0, 0, 0, 127, 0, qo.scale);
    s[mt] = z;
  }
  // logits in the exp2 domain, masked past the visible tokens (a full page,
  // the common case, needs no mask)
  float mx = -INFINITY;
  const bool full = nt >= MPS;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const float kv4[4] = {pr.ks4[mt].x, pr.ks4[mt].y, pr.ks4[mt].z, pr.ks4[mt].w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x = s[mt][v] * (kv4[v] * qscale);
      if (!full) x = (16 * q + 4 * mt + v) < nt ? x : -INFINITY;
      s[mt][v] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  // Lazy rescale: the running reference max moves only when some head's
  // page max exceeds it by more than 2^8 (so p <= 256, no overflow); the
  // output o / l does not depend on the reference.  The first page always
  // sets it (the accumulator is still zero then).
  if (__ballot((lane & 15) < MG && mx > st.m_run + 8.0f)) {   // the 8 real head columns decide
    const float m_new = fmaxf(st.m_run, mx);        // finite: token 0 is visible
    if (st.m_run != -INFINITY) {
      const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
      st.l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) st.acc[dt] *= alpha;
    }
    st.m_run = m_new;
  }
  const float m_ref = st.m_run;
  float psum = 0.f;
  f32x8 pv[2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const float vv4[4] = {pr.vs4[mt].x, pr.vs4[mt].y, pr.vs4[mt].z, pr.vs4[mt].w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float p = __builtin_amdgcn_exp2f(s[mt][v] - m_ref);
      psum += p;
      pv[mt >> 1][4 * (mt & 1) + v] = p * vv4[v];
    }
  }
  psum += __shfl_xor(psum, 16, 64);
  psum += __shfl_xor(psum, 32, 64);
  st.l_run += psum;
  const bf16x8 pb0 = __builtin_convertvector(pv[0], bf16x8);
  const bf16x8 pb1 = __builtin_convertvector(pv[1], bf16x8);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    bf16x8 v0, v1;
    fp8x16_to_bf16(pr.vr[dt], v0, v1);
    f32x4 o = st.acc[dt];
    o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pb0, o, 0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, pb1, o, 0, 0, 0);
    st.acc[dt] = o;
  }
}

// Fold the pages flagged in `mask` (wave-uniform; bit j = lane j's page:
// row pointer rows_lo/hi, visible tokens nt) in ascending lane order,
// loading each page straight into registers (decode: about one page per
// wave).  A page with a write-back row (wb_lo/hi nonzero: read from its
// mirror row) is stored to that pool row's block too.
__device__ __forceinline__ void fold_pages(uint64_t mask, uint32_t rows_lo, uint32_t rows_hi, uint32_t wb_lo,
                                           uint32_t wb_hi, int nt, size_t layer_off, size_t cb, int g, int lane,
                                           QOp& qo, bool& have_q, const uint4 (&qraw)[4], float qscale,
                                           WaveAttn& st) {
  while (mask) {
    const int j = __builtin_ctzll(mask);
    mask &= mask - 1;
    const uint64_t pv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)rows_hi, j) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)rows_lo, j);
    const uint64_t wv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)wb_hi, j) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)wb_lo, j);
    PageRegs cur;
    load_page(reinterpret_cast<const uint8_t*>(pv) + layer_off, cb, g, lane, cur);
    if (wv) store_page(reinterpret_cast<uint8_t*>(wv) + layer_off, cb, g, lane, cur);
    if (!have_q) {                 // built while the first page's loads are in flight
      make_qop(qraw, qo);
      have_q = true;
    }
    fold_page(cur, __builtin_amdgcn_readlane(nt, j), lane, qo, qscale, st);
  }
}

// ---- LDS-staged page pipeline (many pages per wave) ----------------------
// Each wave owns a 17 KiB LDS buffer.  While a page is folded from
// registers, the next page is already streaming into the buffer with
// direct global->LDS 16-byte loads (lane L's bytes land at base + 16 L), so
// a wave keeps a page in flight without registers for it.  The buffer
// holds the page XOR-swizzled so that the operand reads are free of bank
// conflicts: K row t's 16-byte chunk c sits at granule 8t + (c ^ fK(t));
// V^T row r's chunk c at granule 512 + 4r + (c ^ fV(r)); then the K and V
// scales (granules 1024..1055, K then V; lanes 32..63 load a duplicate copy).
constexpr int PBUF = 17408;
__device__ __forceinline__ int fK(int t) { return ((t >> 4) & 3) | ((t & 2) << 1); }
__device__ __forceinline__ int fV(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void stage_page(const uint8_t* blk, size_t cb, int g, int lane, uint8_t* buf) {
  const uint8_t* kb = blk + (size_t)g * MPS * MD;
  const uint8_t* vb = blk + cb + (size_t)g * MPS * MD;
  const uint8_t* sc = blk + 2 * cb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int G = 64 * i + lane, t = G >> 3, ch = (G & 7) ^ fK(t);
    __builtin_amdgcn_global_load_lds((const void*)(kb + t * MD + 16 * ch), buf + 1024 * i, 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int G = 64 * i + lane, r = G >> 2, ch = (G & 3) ^ fV(r);
    __builtin_amdgcn_global_load_lds((const void*)(vb + r * MPS + 16 * ch), buf + 8192 + 1024 * i, 16, 0, 0);
  }
  __builtin_amdgcn_global_load_lds((const void*)(sc + 16 * (lane & 31)), buf + 16384, 16, 0, 0);
}

__device__ __forceinline__ void read_page(const uint8_t* buf, int lane, PageRegs& pr) {
  const int m = lane & 15, q = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int t = 16 * (m >> 2) + 4 * mt + (m & 3), f = fK(t);
    const uint4 k0 = *reinterpret_cast<const uint4*>(buf + 16 * (8 * t + ((2 * q) ^ f)));
    const uint4 k1 = *reinterpret_cast<const uint4*>(buf + 16 * (8 * t + ((2 * q + 1) ^ f)));
    pr.ka[mt] = i32x8{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int r = 16 * dt + m;
    pr.vr[dt] = *reinterpret_cast<const uint4*>(buf + 8192 + 16 * (4 * r + (q ^ fV(r))));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr.ks4[i] = *reinterpret_cast<const float4*>(buf + 16384 + 4 * (16 * q + 4 * i));
    pr.vs4[i] = *reinterpret_cast<const float4*>(buf + 16384 + 4 * MPS + 4 * (16 * q + 4 * i));
  }
}

// As fold_pages, with the next page staged through the wave's LDS buffer.
__device__ __forceinline__ void fold_pages_lds(uint64_t mask, uint32_t rows_lo, uint32_t rows_hi, int nt,
                                               size_t layer_off, size_t cb, int g, int lane, const QOp& qo,
                                               float qscale, WaveAttn& st, uint8_t* buf) {
  if (!mask) return;
  auto row_of = [&](int jj) {
    const uint64_t pv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)rows_hi, jj) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)rows_lo, jj);
    return reinterpret_cast<const uint8_t*>(pv) + layer_off;
  };
  int j = __builtin_ctzll(mask);
  mask &= mask - 1;
  stage_page(row_of(j), cb, g, lane, buf);
  while (true) {
    __builtin_amdgcn_s_waitcnt(0);          // the staged page has landed
    PageRegs cur;
    read_page(buf, lane, cur);
    __builtin_amdgcn_s_waitcnt(0);          // reads done before the buffer is refilled
    const int n = __builtin_amdgcn_readlane(nt, j);
    const bool more = mask != 0;
    if (more) {
      j = __builtin_ctzll(mask);
      mask &= mask - 1;
      stage_page(row_of(j), cb, g, lane, buf);
    }
    fold_page(cur, n, lane, qo, qscale, st);
    if (!more) break;
  }
}

// Selected entry j of row r (request b): local id -> pool slot (or, for the
// host tail, the page's mirror row) and the page's visible tokens (0: none).
// An entry the launch's own fetch brings in is read from its mirror row and
// `wb` is its slot's row (else null).
__device__ __forceinline__ void resolve_page(const DevCtx& c, const AttnArgs& a, int r, int b, int j, int limit,
                                             const uint8_t*& row, int& nt, uint8_t*& wb) {
  row = nullptr;
  nt = 0;
  wb = nullptr;
  const int i = a.sel[(size_t)r * a.topk + j];
  if (a.slots) {
    const size_t idx = (size_t)r * (a.slots_stride > 0 ? a.slots_stride : a.topk) + j;
    const int s = a.slots[idx];
    const int fetched = a.slot_miss ? (int)a.slot_miss[idx] : 0;
    const int pg = fetched ? a.slot_page[idx] : -1;
    if (i >= 0 && s >= 0 && s < c.S) {
      row = c.pool + (size_t)s * c.row_bytes;
      nt = min(MPS, limit - i * MPS);
      if (fetched && pg >= 0 && (int64_t)pg < c.N) {
        wb = c.pool + (size_t)s * c.row_bytes;
        row = c.mirror + (size_t)pg * c.row_bytes;
      }
    }
  } else if (i >= 0 && i < a.max_pages) {
    const int page = a.bt[(size_t)b * a.max_pages + i];
    if (page >= 0 && (int64_t)page < c.N) {
      const int slot = c.page_to_slot[page];
      if (slot >= 0) row = c.pool + (size_t)slot * c.row_bytes;
      else if (a.host_tail) row = c.mirror + (size_t)page * c.row_bytes;
    }
    nt = min(MPS, limit - i * MPS);
  }
  if (!row) nt = 0;
}

// Pages j = jbeg, jbeg + jstep, ... < jend of row r (request b), KV head g.
// The query operand: ready (STAGED) or built by the register path from the
// raw query once the first page's loads are in flight.
template <bool STAGED>
__device__ __forceinline__ void wave_pages(const DevCtx& c, const AttnArgs& a, int r, int b, int g,
                                           int jbeg, int jend, int jstep, int lane,
                                           QOp& qop, bool& have_q, const uint4 (&qraw)[4], WaveAttn& st,
                                           uint8_t* lds) {
  int limit = a.ctx_len[b];
  if (a.row_pos) limit = min(limit, a.row_pos[r] + 1);
  const float qscale = 1.4426950408889634f / sqrtf((float)MD);
  const size_t cb = (size_t)c.code_bytes;
  for (int base = jbeg; base < jend; base += 64 * jstep) {
    // lane i resolves page base + i*jstep: local id -> pool slot (or, for
    // the host tail, the page's mirror row), visible tokens
    const int j = base + lane * jstep;
    const uint8_t* row = nullptr;
    uint8_t* wb = nullptr;
    int nt = 0;
    if (j < jend) resolve_page(c, a, r, b, j, limit, row, nt, wb);
    const uint64_t rowv = reinterpret_cast<uint64_t>(row), wbv = reinterpret_cast<uint64_t>(wb);
    const uint64_t mask = __ballot(nt > 0);
    if constexpr (STAGED)   // (no write-back rows: the launcher folds the fetch into split launches only)
      fold_pages_lds(mask, (uint32_t)rowv, (uint32_t)(rowv >> 32), nt, (size_t)a.layer * c.layer_bytes, cb, g,
                     lane, qop, qscale, st, lds);
    else
      fold_pages(mask, (uint32_t)rowv, (uint32_t)(rowv >> 32), (uint32_t)wbv, (uint32_t)(wbv >> 32), nt,
                 (size_t)a.layer * c.layer_bytes, cb, g, lane, qop, have_q, qraw, qscale, st);
  }
}

__device__ __forceinline__ void init_state(WaveAttn& st) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
}

}  // namespace

// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).  When
// the KV heads divide the XCDs evenly, a workgroup covers consecutive rows
// (one per wave) of one KV head and XCD x only ever serves head x / (8 / Hkv):
// each L2 then caches one head's blocks of the pages instead of all of them.
constexpr int NXCD = 8;

__host__ __device__ __forceinline__ bool attn_rows_by_xcd(int Hkv) { return Hkv <= NXCD && NXCD % Hkv == 0; }

// One wave per (row, KV head), all of the row's pages; RW waves per
// workgroup.  Eight waves in one workgroup (8 LDS page buffers, 136 KiB: one
// workgroup per CU) beat two workgroups of four per CU: on MI355X a 4,096-row
// chunk's attention took 8.52-8.55 ms over 12 layers against 9.15-9.22 ms
// (6 or 7 waves: 9.05-9.24 ms).  A loads-only probe of the same gather gave
// the same ordering (620 against 755 us per layer).
constexpr int RW = 8;
__global__ __launch_bounds__(RW * 64, 2) void k_attn_mfma_rows(DevCtx c, AttnArgs a) {
  __shared__ __align__(16) uint8_t pbuf[RW][PBUF];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int r, g;
  if (attn_rows_by_xcd(c.Hkv)) {
    const int per = NXCD / c.Hkv;                       // XCDs per KV head
    const int x = blockIdx.x % NXCD, k = blockIdx.x / NXCD;
    g = x / per;
    r = (k * per + x % per) * RW + wave;
  } else {
    const int u = blockIdx.x * RW + wave;
    r = u / c.Hkv;
    g = u - r * c.Hkv;
  }
  if (r >= a.rows) return;
  const int b = attn_row_request(a, r);
  QOp qop;
  load_query(a, c, r, g, lane, qop);
  WaveAttn st;
  init_state(st);
  bool have_q = true;
  const uint4 no_raw[4] = {};
  wave_pages<true>(c, a, r, b, g, 0, a.topk, 1, lane, qop, have_q, no_raw, st, pbuf[wave]);
  const int h = lane & 15, q = lane >> 4;
  if (h >= MG) return;
  const float inv = st.l_run > 0.f ? 1.f / st.l_run : 0.f;
  uint16_t* op = a.out + ((size_t)r * c.Hq + g * MG + h) * MD + 4 * q;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const f32x4 o = st.acc[dt] * inv;
    const uint2 w = make_uint2((uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16),
                               (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16));
    *reinterpret_cast<uint2*>(op + 16 * dt) = w;
  }
}

// Page-range passes for many rows (prefill chunks).  Rows select their pages
// all over the request's page space, so a single pass keeps every page of
// every KV head in flight at once and most reads miss the L2s.  Instead the
// attention runs as one launch per range of RP local page ids: in launch r
// each (row, KV head) wave folds in only its selected pages in range r, so
// the pages in flight are one range -- one KV head's blocks of it fit an
// XCD's L2 -- and the online-softmax state (O^T tiles, m, l) is carried
// between launches in an fp32 record per (row, KV head).  Pages are still
// folded in ascending order and the state round-trips exactly, so the result
// is bit-identical to the single pass.  A unit touches the record only
// between its first and last non-empty range: the first starts from an empty
// state, the last writes the bf16 output.
constexpr int ST_FLOATS = ATTN_STATE_FLOATS;   // O^T tiles of the 32 live lanes, then (m, l) per head
static_assert(ST_FLOATS == 8 * 32 * 4 + MG * 2, "record layout");

__global__ __launch_bounds__(TKV_BLOCK, 2) void k_attn_mfma_range(DevCtx c, AttnArgs a, int r, int RP) {
  __shared__ __align__(16) uint8_t pbuf[MWAVES][PBUF];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int row, g;
  if (attn_rows_by_xcd(c.Hkv)) {
    const int per = NXCD / c.Hkv;
    const int x = blockIdx.x % NXCD, k = blockIdx.x / NXCD;
    g = x / per;
    row = (k * per + x % per) * MWAVES + wave;
  } else {
    const int u = blockIdx.x * MWAVES + wave;
    row = u / c.Hkv;
    g = u - row * c.Hkv;
  }
  if (row >= a.rows) return;
  const int b = attn_row_request(a, row);
  int limit = a.ctx_len[b];
  if (a.row_pos) limit = min(limit, a.row_pos[row] + 1);
  // lane j resolves the row's j-th selected page (topk <= 64)
  const uint8_t* base = nullptr;
  int nt = 0, rg = -1;
  if (lane < a.topk) {
    const int i = a.sel[(size_t)row * a.topk + lane];
    if (i >= 0 && i < a.max_pages) {
      const int page = a.bt[(size_t)b * a.max_pages + i];
      if (page >= 0 && (int64_t)page < c.N) {
        const int slot = c.page_to_slot[page];
        if (slot >= 0) base = c.pool + (size_t)slot * c.row_bytes;
        else if (a.host_tail) base = c.mirror + (size_t)page * c.row_bytes;
      }
      nt = min(MPS, limit - i * MPS);
      rg = i / RP;
    }
    if (!base || nt <= 0) {
      nt = 0;
      rg = -1;
    }
  }
  int first = rg >= 0 ? rg : 0x7FFFFFFF, last = rg;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    first = min(first, __shfl_xor(first, o, 64));
    last = max(last, __shfl_xor(last, o, 64));
  }
  const int h = lane & 15, q = lane >> 4;
  uint16_t* op = a.out + ((size_t)row * c.Hq + g * MG + (h < MG ? h : 0)) * MD + 4 * q;
  if (last < 0) {                                       // no page at all: zeros, once
    if (r == 0 && h < MG)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(0u, 0u);
    return;
  }
  if (r < first || r > last) return;
  uint64_t mine = __ballot(rg == r);
  if (!mine) return;                                    // nothing in this range: the record stays
  QOp qop;
  load_query(a, c, row, g, lane, qop);
  float* rec = c.attn_state + ((size_t)row * c.Hkv + g) * ST_FLOATS;
  WaveAttn st;
  init_state(st);
  const int k = q * MG + h;                             // live lane index (h < 8)
  if (r != first) {
    if (h < MG) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) st.acc[dt] = *reinterpret_cast<const f32x4*>(rec + (dt * 32 + k) * 4);
      const float2 ml = *reinterpret_cast<const float2*>(rec + 8 * 32 * 4 + 2 * h);
      st.m_run = ml.x;
      st.l_run = ml.y;
    } else {
      st.m_run = 0.f;   // the zero-query columns' max after any page, as in one pass
    }
  }
  const float qscale = 1.4426950408889634f / sqrtf((float)MD);
  const size_t cb = (size_t)c.code_bytes;
  const uint64_t bv = reinterpret_cast<uint64_t>(base);
  fold_pages_lds(mine, (uint32_t)bv, (uint32_t)(bv >> 32), nt, (size_t)a.layer * c.layer_bytes, cb, g, lane, qop,
                 qscale, st, pbuf[wave]);
  if (h >= MG) return;
  if (r == last) {
    const float inv = st.l_run > 0.f ? 1.f / st.l_run : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 o = st.acc[dt] * inv;
      const uint2 w = make_uint2((uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16),
                                 (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16));
      *reinterpret_cast<uint2*>(op + 16 * dt) = w;
    }
    return;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(rec + (dt * 32 + k) * 4) = st.acc[dt];
  if (q == 0) *reinterpret_cast<float2*>(rec + 8 * 32 * 4 + 2 * h) = make_float2(st.m_run, st.l_run);
}

// a workgroup per (row, KV head, page range); wave w takes every 4th page
// The fetch folded into a split launch: workgroups past the attention's rows
// copy the miss list's rows host -> device, every layer's block but this
// launch's (which the waves that fold those pages write back), in 16 KiB
// items dealt to them in turn, two 16-byte loads in flight per thread.
constexpr int FUSED_FETCH_WGS = 64;
__device__ void attn_fused_fetch(const DevCtx& c, const AttnArgs& a) {
  const int F = (int)gridDim.x * ((int)gridDim.y - a.rows);
  const int f = ((int)blockIdx.y - a.rows) * (int)gridDim.x + (int)blockIdx.x;
  int m = *a.fmiss_count;
  if (m > a.fwidth) m = a.fwidth;
  if (f == 0 && threadIdx.x == 0 && m > 0) c.hdr->counters[CNT_BYTES_FETCHED] += (int64_t)m * c.row_bytes;
  const int64_t nvl = c.layer_bytes / 16, la = (int64_t)a.layer * nvl;
  const int64_t nvec = c.row_bytes / 16 - nvl;          // the row without this layer's block
  constexpr int64_t IV = 1024;                          // vectors per item
  const int64_t ipr = (nvec + IV - 1) / IV;
  const int64_t items = (int64_t)m * ipr;
  for (int64_t it = f; it < items; it += F) {
    const int mi = (int)(it / ipr);
    const int64_t ch = it - (int64_t)mi * ipr;
    const int slot = a.fmiss[2 * mi], page = a.fmiss[2 * mi + 1];
    if (slot < 0 || slot >= c.S || page < 0 || (int64_t)page >= c.N) {
      if (threadIdx.x == 0) set_error(c.hdr, DERR_BAD_MISS);
      continue;
    }
    const u32x4v* src = reinterpret_cast<const u32x4v*>(c.mirror + (size_t)page * c.row_bytes);
    u32x4v* dst = reinterpret_cast<u32x4v*>(c.pool + (size_t)slot * c.row_bytes);
    const int64_t v_end = min(nvec, (ch + 1) * IV);
    for (int64_t v0 = ch * IV + threadIdx.x; v0 < v_end; v0 += 2 * TKV_BLOCK) {
      u32x4v t0, t1;
      const int64_t x0 = v0, x1 = v0 + TKV_BLOCK;
      const int64_t r0 = x0 >= la ? x0 + nvl : x0, r1 = x1 >= la ? x1 + nvl : x1;
      t0 = __builtin_nontemporal_load(src + r0);
      if (x1 < v_end) t1 = __builtin_nontemporal_load(src + r1);
      dst[r0] = t0;
      if (x1 < v_end) dst[r1] = t1;
    }
  }
}

__global__ __launch_bounds__(TKV_BLOCK) void k_attn_mfma_split(DevCtx c, AttnArgs a) {
  __shared__ __align__(16) float sO[MWAVES][MG][MD];
  __shared__ float sM[MWAVES][MG], sL[MWAVES][MG];
  __shared__ int sflag[2];
  if ((int)blockIdx.y >= a.rows) {   // (only with a folded fetch)
    attn_fused_fetch(c, a);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.y;
  const int g = blockIdx.x % c.Hkv;
  const int split = blockIdx.x / c.Hkv;
  const int j0 = split * a.pages_per_split;
  const int j1 = min(a.topk, j0 + a.pages_per_split);
  const int b = attn_row_request(a, r);
  uint4 qraw[4];
  load_query_raw(a, c, r, g, lane, qraw);
  QOp qop;
  bool have_q = false;
  WaveAttn st;
  init_state(st);
  wave_pages<false>(c, a, r, b, g, j0 + wave, j1, MWAVES, lane, qop, have_q, qraw, st, nullptr);
  const int h = lane & 15, q = lane >> 4;
  if (h < MG) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(&sO[wave][h][16 * dt + 4 * q]) =
          make_float4(st.acc[dt][0], st.acc[dt][1], st.acc[dt][2], st.acc[dt][3]);
    if (q == 0) {
      sM[wave][h] = st.m_run;
      sL[wave][h] = st.l_run;
    }
  }
  __syncthreads();
  // merge the waves: thread = (head, 4 d values)
  const int hh = tid / 32, d0 = (tid % 32) * 4;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < MWAVES; ++w) M = fmaxf(M, sM[w][hh]);
  float L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < MWAVES; ++w) {
      const float mw = sM[w][hh];
      const float wt = mw == -INFINITY ? 0.f : exp2f(mw - M);
      const float4 ow = *reinterpret_cast<const float4*>(&sO[w][hh][d0]);
      L += sL[w][hh] * wt;
      o.x += ow.x * wt; o.y += ow.y * wt; o.z += ow.z * wt; o.w += ow.w * wt;
    }
  }
  if (a.splits == 1) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* op = a.out + ((size_t)r * c.Hq + g * MG + hh) * MD + d0;
    op[0] = f32_to_bf16(o.x * inv); op[1] = f32_to_bf16(o.y * inv);
    op[2] = f32_to_bf16(o.z * inv); op[3] = f32_to_bf16(o.w * inv);
    return;
  }
  float* rec = c.attn_part + (((size_t)r * c.Hq + g * MG + hh) * a.splits + split) * ATT_REC;
  *reinterpret_cast<float4*>(rec + d0) = o;
  if (d0 == 0) *reinterpret_cast<float2*>(rec + MD) = make_float2(M, L);
  if (!last_block_arrive(&c.attn_done[r * c.Hkv + g], a.splits, &sflag[0])) return;
  attn_merge_splits(c, a, r, g, tid);
}

bool attn_mfma_supported(const DevCtx& c) {
  return c.fp8 && c.PS == MPS && c.D == MD && c.Hq == MG * c.Hkv;
}

hipError_t launch_attn_mfma(const DevCtx& c, AttnArgs a, hipStream_t st) {
  if (!attn_mfma_supported(c)) return hipErrorInvalidValue;
  const long units = (long)a.rows * c.Hkv;
  if (a.rows > c.max_batch || units >= 256) {
    if (a.fmiss || a.slot_miss) return hipErrorInvalidValue;   // a folded fetch: split launches only
    a.splits = 1;
    a.pages_per_split = a.topk;
    // workgroups of `w` waves, one (row, KV head) each; with the XCD mapping
    // each KV head takes groups of w rows on its own XCDs
    auto grid_of = [&](int w) {
      if (!attn_rows_by_xcd(c.Hkv)) return (int)((units + w - 1) / w);
      const int per = NXCD / c.Hkv;
      const int groups = (a.rows + w - 1) / w;             // row groups per head
      return NXCD * ((groups + per - 1) / per);
    };
    const int RP = c.attn_range_pages;
    if (RP > 0 && c.attn_state && a.topk <= 64 && a.rows <= c.max_rows && a.max_pages > RP) {
      const int blocks = grid_of(MWAVES);
      const int nr = (a.max_pages + RP - 1) / RP;
      for (int r = 0; r < nr; ++r) {
        hipLaunchKernelGGL(k_attn_mfma_range, dim3(blocks), dim3(TKV_BLOCK), 0, st, c, a, r, RP);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
    hipLaunchKernelGGL(k_attn_mfma_rows, dim3(grid_of(RW)), dim3(RW * 64), 0, st, c, a);
    return hipGetLastError();
  }
  // one page per wave; a folded fetch adds rows of workgroups past a.rows
  a.pages_per_split = MWAVES;
  a.splits = (a.topk + MWAVES - 1) / MWAVES;
  const int gx = c.Hkv * a.splits;
  const int fy = a.fmiss ? (FUSED_FETCH_WGS + gx - 1) / gx : 0;
  dim3 grid(gx, a.rows + fy);
  hipLaunchKernelGGL(k_attn_mfma_split, grid, dim3(TKV_BLOCK), 0, st, c, a);
  return hipGetLastError();
}

bool attn_mfma_split_applies(const DevCtx& c, int rows) {
  return c.attn_impl != ATTN_VECTOR && attn_mfma_supported(c) && rows <= c.max_batch && (long)rows * c.Hkv < 256;
}
