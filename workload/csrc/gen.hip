// Seeded input generator, GPU side: the same Philox4x64-10 block stream as
// NumPy's Philox bit generator (Salmon, Moraes, Dror, Shaw, SC 2011), mapped
// through the same 65,536-entry grid table.  Input generation only -- nothing
// here computes any step of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

struct u64x4 { uint64_t v[4]; };

__device__ __forceinline__ u64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                               uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B97F4A7C15ull;
    k1 += 0xBB67AE8584CAA73Bull;
  }
  u64x4 o;
  o.v[0] = c0; o.v[1] = c1; o.v[2] = c2; o.v[3] = c3;
  return o;
}

// Tokens [start, start+count) of one request in one layer, bf16 [count][H][D].
// exp2neg >= 0: the table holds grid integers m, value m * 2^-exp2neg;
// exp2neg < 0: the table holds the bf16 bit patterns themselves.
// Block b of `block_tokens` tokens uses key (seed<<16 | kind, layer<<48 | req<<32 | b);
// within a block the i-th 16-bit uniform is half (i%4) of 64-bit word (i/4)%4 of
// Philox(counter = i/16 + 1).
__global__ void k_gen_tokens(uint16_t* out, const int16_t* table, int exp2neg, uint64_t seed, int kind,
                             int layer, int req, int start, int count, int block_tokens, int HD) {
  const int64_t per_block = (int64_t)block_tokens * HD;
  const int b0 = start / block_tokens, b1 = (start + count - 1) / block_tokens;
  const int64_t groups_per_block = per_block / 16;
  const int64_t total = (int64_t)(b1 - b0 + 1) * groups_per_block;
  const float scale = ldexpf(1.0f, -exp2neg);
  for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < total;
       gi += (int64_t)gridDim.x * blockDim.x) {
    const int blk = b0 + (int)(gi / groups_per_block);
    const int64_t ci = gi % groups_per_block;
    const int64_t first = (int64_t)blk * per_block + ci * 16;  // value index within the request
    const int64_t lo = (int64_t)start * HD, hi = (int64_t)(start + count) * HD;
    if (first + 16 <= lo || first >= hi) continue;
    const uint64_t k0 = (seed << 16) | (uint64_t)kind;
    const uint64_t k1 = ((uint64_t)layer << 48) | ((uint64_t)req << 32) | (uint64_t)blk;
    const u64x4 r = philox4x64_10((uint64_t)ci + 1, 0, 0, 0, k0, k1);
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int64_t vi = first + w * 4 + h;
        if (vi < lo || vi >= hi) continue;
        const uint32_t u = (uint32_t)(r.v[w] >> (16 * h)) & 0xFFFFu;
        if (exp2neg < 0) {
          out[vi - lo] = (uint16_t)table[u];
        } else {
          const float x = (float)table[u] * scale;
          out[vi - lo] = (uint16_t)(__float_as_uint(x) >> 16);
        }
      }
  }
}

extern "C" int tkvgen_tokens(uint16_t* out, const int16_t* table, int exp2neg, uint64_t seed, int kind,
                             int layer, int req, int start, int count, int block_tokens, int HD,
                             void* stream) {
  if (count <= 0) return 0;
  const int64_t per_block = (int64_t)block_tokens * HD;
  if (per_block % 16) return -1;
  const int nb = (start + count - 1) / block_tokens - start / block_tokens + 1;
  int64_t groups = (int64_t)nb * per_block / 16;
  int grid = (int)((groups + 255) / 256);
  if (grid > 16384) grid = 16384;
  hipLaunchKernelGGL(k_gen_tokens, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, table, exp2neg,
                     seed, kind, layer, req, start, count, block_tokens, HD);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
