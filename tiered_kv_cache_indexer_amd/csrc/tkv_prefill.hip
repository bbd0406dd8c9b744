// Indexer scores of a prefill chunk on the matrix cores (gfx950).
//
// FreeToken PR #499, "Why this works for sparse attention": the indexer
// scores pages on the GPU-resident compressed slab before any page is read.
// For a chunk of query rows of one request this is a dense product: the
// per-group query sums qg [rows][Hkv*d] (bf16) times the slab rows of the
// request's pages [pages][Hkv*d] (bf16, gathered through the block table).
//
// k_group_q forms qg = bf16(exact sum of the group's query heads): the fp64
// sum of 8 bf16 values is exact, and so is its conversion to fp32 for values
// on the query grid, so the bf16 rounding is the only one.
// k_prefill_scores: one 256-thread workgroup per 64 rows x 64 pages; each wave
// owns 32 x 32 outputs as 2 x 2 tiles of v_mfma_f32_16x16x32_bf16.  Lane i of
// a wave reads row (i % 16) of a 16 x 32 A tile and page (i % 16) of the
// 32 x 16 B tile from LDS, 8 consecutive features (16 bytes) at feature
// offset 8 * (i / 16): A and B use the same feature slicing, so the product
// is the dot product over all features.  Accumulation is fp32; with the inputs on
// the indexer grids (qg on 2^-5, slab on 2^-10, sum |qg*slab| < 2^9) every
// partial sum is exact, so the scores equal the decode scan's bit for bit.
#include "tkv_dev.h"
#include "tkv_launch.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// thread = 8 consecutive features of one row's group sum (16-byte loads)
__global__ __launch_bounds__(TKV_BLOCK) void k_group_q(DevCtx c, const uint16_t* q, int rows, uint16_t* qg) {
  const int G = c.Hq / c.Hkv, E = c.Hkv * c.D;
  const int per_row = E / 8;
  const int t = blockIdx.x * TKV_BLOCK + threadIdx.x;
  const int r = t / per_row, e0 = (t - r * per_row) * 8;
  if (r >= rows) return;
  const int g = e0 / c.D, dd = e0 - g * c.D;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  for (int h = 0; h < G; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(q + ((size_t)r * c.Hq + g * G + h) * c.D + dd);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += (double)__uint_as_float(ww[i] << 16);
      acc[2 * i + 1] += (double)__uint_as_float(ww[i] & 0xFFFF0000u);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)f32_to_bf16((float)acc[2 * i]) | ((uint32_t)f32_to_bf16((float)acc[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(qg + (size_t)r * E + e0) = make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, w);
}

template <int E>
__global__ __launch_bounds__(TKV_BLOCK) void k_prefill_scores(DevCtx c, SelArgs a, const uint16_t* qg) {
  // The workgroup's 64 query rows and 64 pages pass through LDS in chunks of
  // 64 features (128 bytes of a row): a load instruction moves whole 128-byte
  // row pieces (8 rows a wave), each row is read from the caches once per
  // workgroup instead of once per wave, and the next chunk's loads are in
  // flight while the current one is multiplied.  Rows are padded to 144
  // bytes, so the fragment reads (16 rows, 16 bytes each) hit distinct banks.
  constexpr int KC = 64, NCH = E / KC, RS = KC * 2 + 16;
  __shared__ __align__(16) uint8_t lds[2][2][64 * RS];   // [buffer][query rows | pages]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int rowb = blockIdx.y * 64, pb = blockIdx.x * 64;
  const int row0 = rowb + wr * 32;
  const int p0 = pb + wc * 32;
  const int m = lane & 15, kq = lane >> 4;
  const int npg = min(a.n_pages[0], a.max_pages);
  const uint16_t* slab_l = c.slab + (size_t)a.layer * c.N * E;

  // loader: thread t moves 16-byte piece t % 8 of rows t / 8 and t / 8 + 32
  // (a page outside the request loads slab row 0; its column is set to -inf)
  const int lp = tid & 7, lr = tid >> 3;
  const uint16_t* asrc[2];
  const uint16_t* bsrc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = min(rowb + lr + 32 * h, a.rows - 1);
    asrc[h] = qg + (size_t)r * E + lp * 8;
    const int p = pb + lr + 32 * h;
    int lg = p < npg ? a.bt[p] : -1;
    if (!(lg >= 0 && (int64_t)lg < c.N)) lg = 0;
    bsrc[h] = slab_l + (size_t)lg * E + lp * 8;
  }
  // this lane's output pages
  int logical[2];
  bool bok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int p = p0 + t * 16 + m;
    int lg = -1;
    if (p < npg) lg = a.bt[p];
    bok[t] = lg >= 0 && (int64_t)lg < c.N;
    logical[t] = bok[t] ? lg : 0;
  }
  const uint4* a0 = reinterpret_cast<const uint4*>(asrc[0]);
  const uint4* a1 = reinterpret_cast<const uint4*>(asrc[1]);
  const uint4* b0 = reinterpret_cast<const uint4*>(bsrc[0]);
  const uint4* b1 = reinterpret_cast<const uint4*>(bsrc[1]);
  const int so0 = lr * RS + lp * 16, so1 = (lr + 32) * RS + lp * 16;
  constexpr int CV = KC / 8;   // 16-byte vectors per chunk of a row
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 ra0 = a0[0], ra1 = a1[0], rb0 = b0[0], rb1 = b1[0];
  *reinterpret_cast<uint4*>(&lds[0][0][so0]) = ra0;
  *reinterpret_cast<uint4*>(&lds[0][0][so1]) = ra1;
  *reinterpret_cast<uint4*>(&lds[0][1][so0]) = rb0;
  *reinterpret_cast<uint4*>(&lds[0][1][so1]) = rb1;
  __syncthreads();
#pragma unroll 2
  for (int ch = 0; ch < NCH; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < NCH) {
      ra0 = a0[(ch + 1) * CV];
      ra1 = a1[(ch + 1) * CV];
      rb0 = b0[(ch + 1) * CV];
      rb1 = b1[(ch + 1) * CV];
    }
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&lds[buf][0][(wr * 32 + t * 16 + m) * RS + s * 64 + kq * 16]));
        bv[t] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&lds[buf][1][(wc * 32 + t * 16 + m) * RS + s * 64 + kq * 16]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (ch + 1 < NCH) {   // nobody reads buffer buf ^ 1 until the barrier below
      *reinterpret_cast<uint4*>(&lds[buf ^ 1][0][so0]) = ra0;
      *reinterpret_cast<uint4*>(&lds[buf ^ 1][0][so1]) = ra1;
      *reinterpret_cast<uint4*>(&lds[buf ^ 1][1][so0]) = rb0;
      *reinterpret_cast<uint4*>(&lds[buf ^ 1][1][so1]) = rb1;
    }
    __syncthreads();
  }
  // output tile (i, j): lane holds rows 4*(lane/16) + v, page column lane % 16
  float bias[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) bias[j] = (a.bias && bok[j]) ? a.bias[logical[j]] : 0.f;
  float* __restrict__ sc = c.scores;
  // interior tiles (a wave-uniform test) store without per-lane conditions,
  // so the 16 stores issue back to back
  float key[2][2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) key[j][i][v] = bok[j] ? acc[i][j][v] + bias[j] : -INFINITY;
  float* base = sc + (size_t)(row0 + kq * 4) * c.max_pages + p0 + m;
  if (p0 + 32 <= npg && row0 + 32 <= a.rows) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) base[(size_t)(i * 16 + v) * c.max_pages + j * 16] = key[j][i][v];
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (p0 + j * 16 + m < npg && row0 + i * 16 + kq * 4 + v < a.rows)
            base[(size_t)(i * 16 + v) * c.max_pages + j * 16] = key[j][i][v];
  }
}

hipError_t launch_prefill_scores(const DevCtx& c, const SelArgs& a, hipStream_t st) {
  uint16_t* qg = c.qg;
  const long threads = (long)a.rows * (c.Hkv * c.D / 8);
  hipLaunchKernelGGL(k_group_q, dim3((unsigned)((threads + TKV_BLOCK - 1) / TKV_BLOCK)), dim3(TKV_BLOCK), 0, st, c,
                     a.q, a.rows, qg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((a.max_pages + 63) / 64, (a.rows + 63) / 64);
  const int E = c.Hkv * c.D;
  if (E == 512) hipLaunchKernelGGL(k_prefill_scores<512>, grid, dim3(TKV_BLOCK), 0, st, c, a, qg);
  else if (E == 128) hipLaunchKernelGGL(k_prefill_scores<128>, grid, dim3(TKV_BLOCK), 0, st, c, a, qg);
  else if (E == 256) hipLaunchKernelGGL(k_prefill_scores<256>, grid, dim3(TKV_BLOCK), 0, st, c, a, qg);
  else if (E == 1024) hipLaunchKernelGGL(k_prefill_scores<1024>, grid, dim3(TKV_BLOCK), 0, st, c, a, qg);
  else return hipErrorInvalidValue;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select_rows(c, a, st);
}
