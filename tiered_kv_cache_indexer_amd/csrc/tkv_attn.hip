// Sparse paged attention over the selected pages (gfx950).
//
// FreeToken PR #499, "Design": after the ensure the block table is
// translated logical->physical and the sparse paged attention reads only the
// selected pages; "Why this works for sparse attention": cold pages are never
// read.  vLLM RFC #33980, "Proposed Change": attention over the top-k KV.
//
// Launch: grid (Hkv * splits, rows), 256 threads.  A workgroup owns one KV
// head (its 8 query heads, GQA) of one row and a contiguous range of the
// row's selected pages, and runs an online softmax over them:
//  * QK: thread = (token, part of d); the part's slice of all 8 query heads
//    lives in registers, the K codes come straight from HBM (16-byte loads),
//    are decoded by the hardware fp8 converter, dotted, reduced over the
//    parts with lane shuffles and scaled by the token's K scale;
//  * softmax: one wave per two heads, exp2 domain (log2(e)/sqrt(d) folded
//    into the query), the token's V scale folded into its probability;
//  * PV: thread = (d, half of the tokens), V codes (fp8: stored transposed,
//    [d][page]) staged in LDS by 16-byte loads, 8 head accumulators per thread.
// With several splits per (row, KV head) each split writes (o, m, l) and the
// last split to finish (atomic counter) merges them and writes bf16 output.
#include "tkv_dev.h"
#include "tkv_launch.h"
#include "tkv_attn_dev.h"





#define ATT_MAXP 64   // pages one workgroup resolves at once

template <int PS, bool FP8>
__global__ __launch_bounds__(TKV_BLOCK) void k_attn(DevCtx c, AttnArgs a) {
  constexpr int D = ATT_D, G = ATT_G;
  constexpr int PARTS = (PS == 64) ? 8 : 16;            // lanes per token in QK
  constexpr int DPP = D / PARTS;                         // d values per part
  constexpr int TOK_PER_PASS = TKV_BLOCK / PARTS;
  constexpr int PASSES = PS / TOK_PER_PASS;
  constexpr int ELT = FP8 ? 1 : 2;
  constexpr int VBYTES = PS * D * ELT;

  __shared__ __align__(16) uint8_t sV[VBYTES];
  __shared__ float sKs[PS], sVs[PS];
  __shared__ float sS[G][PS];
  __shared__ __align__(16) float sP[PS][G];
  __shared__ float sAlpha[G], sM[G], sL[G];
  __shared__ const uint8_t* sBase[ATT_MAXP];
  __shared__ int sNtok[ATT_MAXP];
  __shared__ int sb;
  __shared__ int sflag[2];
  __shared__ __align__(16) float sRed[G][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.y;
  const int g = blockIdx.x % c.Hkv;
  const int split = blockIdx.x / c.Hkv;
  const int j0 = split * a.pages_per_split;
  const int j1 = min(a.topk, j0 + a.pages_per_split);
  const int np = max(0, j1 - j0);

  if (tid == 0) {
    int b = 0;
    while (b + 1 < a.B && a.row_start[b + 1] <= r) ++b;
    sb = b;
  }
  __syncthreads();
  const int b = sb;
  int limit = a.ctx_len[b];
  if (a.row_pos) limit = min(limit, a.row_pos[r] + 1);

  // resolve the split's pages: local id -> logical -> pool slot (or, for the
  // host tail, the page's mirror row), visible tokens
  for (int jj = tid; jj < np && jj < ATT_MAXP; jj += TKV_BLOCK) {
    const int i = a.sel[(size_t)r * a.topk + j0 + jj];
    const uint8_t* base = nullptr;
    int nt = 0;
    if (a.slots) {
      const int s = a.slots[(size_t)r * (a.slots_stride > 0 ? a.slots_stride : a.topk) + j0 + jj];
      if (i >= 0 && s >= 0 && s < c.S) {
        base = c.pool + (size_t)s * c.row_bytes;
        nt = min(PS, limit - i * PS);
      }
    } else if (i >= 0 && i < a.max_pages) {
      const int page = a.bt[(size_t)b * a.max_pages + i];
      if (page >= 0 && (int64_t)page < c.N) {
        const int slot = c.page_to_slot[page];
        if (slot >= 0) base = c.pool + (size_t)slot * c.row_bytes;
        else if (a.host_tail) base = c.mirror + (size_t)page * c.row_bytes;
      }
      nt = min(PS, limit - i * PS);
    }
    sBase[jj] = base;
    sNtok[jj] = (base && nt > 0) ? nt : 0;
  }

  // query slice in registers, pre-scaled for exp2
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  const int part = tid % PARTS, tbase = tid / PARTS;
  float qr[G][DPP];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint16_t* qh = a.q + ((size_t)r * c.Hq + g * G + h) * D + part * DPP;
#pragma unroll
    for (int i = 0; i < DPP; i += 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(qh + i);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        qr[h][i + 2 * t] = __uint_as_float(ww[t] << 16) * qscale;
        qr[h][i + 2 * t + 1] = __uint_as_float(ww[t] & 0xFFFF0000u) * qscale;
      }
    }
  }
  // running softmax state: wave w owns heads 2w, 2w+1
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const int dcol = tid % D, half = tid / D;
  float acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.f;
  __syncthreads();

  for (int jj = 0; jj < np && jj < ATT_MAXP; ++jj) {
    const int nt = sNtok[jj];
    if (nt <= 0) continue;  // uniform
    const uint8_t* blk = sBase[jj] + (size_t)a.layer * c.layer_bytes;
    const uint8_t* kb = blk + (size_t)g * PS * D * ELT;
    const uint8_t* vb = blk + (size_t)c.code_bytes + (size_t)g * PS * D * ELT;
    // stage V codes and the scales
    for (int o = tid * 16; o < VBYTES; o += TKV_BLOCK * 16)
      *reinterpret_cast<uint4*>(sV + o) = *reinterpret_cast<const uint4*>(vb + o);
    if (FP8) {
      const float* ks = reinterpret_cast<const float*>(blk + 2 * (size_t)c.code_bytes);
      for (int t = tid; t < PS; t += TKV_BLOCK) {
        sKs[t] = ks[t];
        sVs[t] = ks[PS + t];
      }
    }
    // QK
    float dot[PASSES][G];
#pragma unroll
    for (int ps_ = 0; ps_ < PASSES; ++ps_) {
      const int tk = tbase + ps_ * TOK_PER_PASS;
      float kf[DPP];
      constexpr int KW = DPP * ELT / 4;                 // 32-bit words per thread per token
      const uint8_t* kp = kb + ((size_t)tk * D + part * DPP) * ELT;
      uint32_t kw[KW];
      if constexpr (KW % 4 == 0) {
#pragma unroll
        for (int v = 0; v < KW / 4; ++v) {
          const uint4 w = reinterpret_cast<const uint4*>(kp)[v];
          kw[4 * v] = w.x; kw[4 * v + 1] = w.y; kw[4 * v + 2] = w.z; kw[4 * v + 3] = w.w;
        }
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(kp);
        kw[0] = w.x; kw[1] = w.y;
      }
      if (FP8) {
#pragma unroll
        for (int t = 0; t < KW; ++t) {
          const f32x2 lo = e4m3x2_lo(kw[t]);
          const f32x2 hi = e4m3x2_hi(kw[t]);
          kf[4 * t] = lo.x; kf[4 * t + 1] = lo.y; kf[4 * t + 2] = hi.x; kf[4 * t + 3] = hi.y;
        }
      } else {
#pragma unroll
        for (int t = 0; t < KW; ++t) {
          kf[2 * t] = __uint_as_float(kw[t] << 16);
          kf[2 * t + 1] = __uint_as_float(kw[t] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < DPP; ++i) s = fmaf(qr[h][i], kf[i], s);
        dot[ps_][h] = s;
      }
    }
#pragma unroll
    for (int ps_ = 0; ps_ < PASSES; ++ps_)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int o = PARTS / 2; o > 0; o >>= 1) dot[ps_][h] += __shfl_xor(dot[ps_][h], o, 64);
    __syncthreads();  // sKs ready
#pragma unroll
    for (int ps_ = 0; ps_ < PASSES; ++ps_) {
      const int tk = tbase + ps_ * TOK_PER_PASS;
      if (part < G) {
        float v = dot[ps_][0];
#pragma unroll
        for (int h = 1; h < G; ++h) v = (part == h) ? dot[ps_][h] : v;
        if (FP8) v *= sKs[tk];
        sS[part][tk] = (tk < nt) ? v : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax, wave w: heads 2w, 2w+1
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int h = 2 * wave + hh;
      const float s = (lane < PS) ? sS[h][lane] : -INFINITY;
      const float mp = wave_max(s);
      const float m_new = fmaxf(m_run[hh], mp);
      const float p = exp2f(s - m_new);
      const float psum = wave_sum(p);
      const float alpha = exp2f(m_run[hh] - m_new);
      l_run[hh] = l_run[hh] * alpha + psum;
      m_run[hh] = m_new;
      if (lane < PS) sP[lane][h] = FP8 ? p * sVs[lane] : p;
      if (lane == 0) sAlpha[h] = alpha;
    }
    __syncthreads();
    // PV
    float al[G];
#pragma unroll
    for (int h = 0; h < G; ++h) al[h] = sAlpha[h];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] *= al[h];
    const int tb = half * (PS / 2), te = tb + PS / 2;
    for (int t = tb; t < te; ++t) {
      float vv;
      if (FP8) {
        const uint32_t code = sV[dcol * PS + t];   // fp8 V is stored transposed [d][page]
        vv = e4m3x2_lo(code).x;
      } else {
        vv = bf16_to_f32(reinterpret_cast<const uint16_t*>(sV)[t * D + dcol]);
      }
      const float4 p0 = *reinterpret_cast<const float4*>(&sP[t][0]);
      const float4 p1 = *reinterpret_cast<const float4*>(&sP[t][4]);
      acc[0] = fmaf(p0.x, vv, acc[0]); acc[1] = fmaf(p0.y, vv, acc[1]);
      acc[2] = fmaf(p0.z, vv, acc[2]); acc[3] = fmaf(p0.w, vv, acc[3]);
      acc[4] = fmaf(p1.x, vv, acc[4]); acc[5] = fmaf(p1.y, vv, acc[5]);
      acc[6] = fmaf(p1.z, vv, acc[6]); acc[7] = fmaf(p1.w, vv, acc[7]);
    }
    __syncthreads();  // before the next page overwrites sV / sP
  }

  // merge the two token halves; publish m, l
  if (half == 1)
#pragma unroll
    for (int h = 0; h < G; ++h) sRed[h][dcol] = acc[h];
  if (lane == 0) {
    sM[2 * wave] = m_run[0]; sM[2 * wave + 1] = m_run[1];
    sL[2 * wave] = l_run[0]; sL[2 * wave + 1] = l_run[1];
  }
  __syncthreads();
  if (half == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] += sRed[h][dcol];

  if (a.splits == 1) {
    if (half == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float l = sL[h];
        const float o = l > 0.f ? acc[h] / l : 0.f;
        a.out[((size_t)r * c.Hq + g * G + h) * D + dcol] = f32_to_bf16(o);
      }
    }
    return;
  }
  // partial record: [r][h][split] -> o[D], m, l (16-byte aligned records)
  constexpr int REC = D + 4;
  if (half == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* rec = c.attn_part + (((size_t)r * c.Hq + g * G + h) * a.splits + split) * REC;
      rec[dcol] = acc[h];
      if (dcol == 0) { rec[D] = sM[h]; rec[D + 1] = sL[h]; }
    }
  }
  if (!last_block_arrive(&c.attn_done[r * c.Hkv + g], a.splits, &sflag[0])) return;
  attn_merge_splits(c, a, r, g, tid);
}

hipError_t launch_attn(const DevCtx& c, AttnArgs a, hipStream_t st) {
  if (c.attn_impl != ATTN_VECTOR && attn_mfma_supported(c)) return launch_attn_mfma(c, a, st);
  if (c.attn_impl == ATTN_MATRIX) return hipErrorInvalidValue;
  if (a.fmiss || a.slot_miss) return hipErrorInvalidValue;   // a folded fetch: matrix-core split launches only
  // splits: enough workgroups to cover the chip for small batches; one split
  // (no merge) when rows exceed the merge scratch (prefill chunks)
  int per = 1;
  if (a.rows > c.max_batch) per = a.topk;
  else {
    const long units = (long)a.rows * c.Hkv * a.topk;
    if (units > 1024) per = (int)((units + 1023) / 1024);
  }
  if (per > ATT_MAXP) per = ATT_MAXP;
  if (per < 1) per = 1;
  a.pages_per_split = per;
  a.splits = (a.topk + per - 1) / per;
  if (a.splits > 1 && a.rows > c.max_batch) return hipErrorInvalidValue;
  dim3 grid(c.Hkv * a.splits, a.rows);
  if (c.PS == 64 && c.fp8) hipLaunchKernelGGL((k_attn<64, true>), grid, dim3(TKV_BLOCK), 0, st, c, a);
  else if (c.PS == 64 && !c.fp8) hipLaunchKernelGGL((k_attn<64, false>), grid, dim3(TKV_BLOCK), 0, st, c, a);
  else if (c.PS == 16 && c.fp8) hipLaunchKernelGGL((k_attn<16, true>), grid, dim3(TKV_BLOCK), 0, st, c, a);
  else if (c.PS == 16 && !c.fp8) hipLaunchKernelGGL((k_attn<16, false>), grid, dim3(TKV_BLOCK), 0, st, c, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
