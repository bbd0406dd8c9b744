// Shared pieces of the two attention kernels (vector and matrix-core).
//
// Partial records: when the selected pages of a (row, KV head) are split
// over several workgroups, each writes, per query head, the unnormalised
// output o[d] = sum_t exp2(s_t - m) v_t, the running max m and the sum
// l = sum_t exp2(s_t - m) (scores in the exp2 domain: log2(e)/sqrt(d) folded
// in) into attn_part[row][q head][split][d + 4].  The last workgroup to
// arrive (atomic counter per (row, KV head)) combines them: with
// M = max m_s, w_s = exp2(m_s - M), out = sum_s w_s o_s / sum_s w_s l_s.
// This is the usual log-sum-exp merge of a softmax over a union of disjoint
// token sets (FreeToken PR #499, "Design": attention over the selected
// pages only; vLLM RFC #33980, "Proposed Change": attention over the top-k).
#pragma once
#include "tkv_dev.h"

#define ATT_D 128
#define ATT_G 8
#define ATT_REC (ATT_D + 4)

// Merge a (row r, KV head g)'s split records and write the bf16 output.
// Called by all 256 threads of the last workgroup: thread = (head, 4 d).
// Every load of a pass is independent, so one pass is one memory round trip.
__device__ __forceinline__ void attn_merge_splits(const DevCtx& c, const AttnArgs& a, int r, int g, int tid) {
  constexpr int D = ATT_D, G = ATT_G, REC = ATT_REC;
  const int h = tid / 32, d0 = (tid % 32) * 4;
  const float* base = c.attn_part + ((size_t)r * c.Hq + g * G + h) * a.splits * REC;
  const int S = a.splits;
  // one pass: a batch of up to 16 records (output slice, max, sum) is loaded
  // at once and folded into a running max; up to 16 splits take one round
  // trip to memory and the same arithmetic as a max pass followed by a sum
  float M = -INFINITY, L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += 16) {
    float4 ov[16];
    float2 ml[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (s0 + u < S) {
        const float* rec = base + (size_t)(s0 + u) * REC;
        ov[u] = *reinterpret_cast<const float4*>(rec + d0);
        ml[u] = *reinterpret_cast<const float2*>(rec + D);
      } else {
        ov[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        ml[u] = make_float2(-INFINITY, 0.f);
      }
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < 16; ++u) Mb = fmaxf(Mb, ml[u].x);
    if (Mb == -INFINITY) continue;
    if (M != -INFINITY && M != Mb) {
      const float sc = exp2f(M - Mb);
      L *= sc;
      o.x *= sc; o.y *= sc; o.z *= sc; o.w *= sc;
    }
    M = Mb;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float w = (ml[u].x == -INFINITY) ? 0.f : exp2f(ml[u].x - M);
      L += ml[u].y * w;
      o.x += ov[u].x * w; o.y += ov[u].y * w; o.z += ov[u].z * w; o.w += ov[u].w * w;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* op = a.out + ((size_t)r * c.Hq + g * G + h) * D + d0;
  op[0] = f32_to_bf16(o.x * inv); op[1] = f32_to_bf16(o.y * inv);
  op[2] = f32_to_bf16(o.z * inv); op[3] = f32_to_bf16(o.w * inv);
}

// Request of row r: the last b with row_start[b] <= r.
__device__ __forceinline__ int attn_row_request(const AttnArgs& a, int r) {
  if (a.one_row_each) return r;
  int b = 0;
  while (b + 1 < a.B && a.row_start[b + 1] <= r) ++b;
  return b;
}
