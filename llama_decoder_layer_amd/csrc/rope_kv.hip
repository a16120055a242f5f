// RoPE on q and k, then the new k and v written into the paged KV cache.
//
// Rotation: pages "LLama" (hotelren.com/news/2693952, section
// "4 LlamaAttention": rotary_emb applied to q and k) and "vLLM Llama 代码解析"
// (yeyulingfeng.com/a/605382, section "4.LlamaAttention": v takes no part).
// The pair (i, i + d/2) of a head at position p turns by p * w_i; cos and
// sin come from the table built in double precision at create time.  The
// rotation is computed in fp32 as
//     y0 = fmaf(x0, c, -(x1 * s)),   y1 = fmaf(x1, c, x0 * s)
// and rounded once to the layer dtype.
//
// Cache write: "模型库与算子层 — 代码走读" (vllm-learning.pages.dev, section
// "Attention 层"): the new k, v are stored before attention reads the cache.
// Position p of sequence b lives in block block_table[b][p / 16], slot
// p % 16: K plane [blocks][kv_heads][16][head_dim], V plane
// [blocks][kv_heads][head_dim][16].  V is a bit copy of the projection's v.
//
// HBM-bound and tiny: one workgroup per token.  q is rotated in place inside
// the qkv buffer.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_kv_kernel(T* __restrict__ qkv, const int* __restrict__ positions,
                                                      const float2* __restrict__ table, int nq, int nkv,
                                                      int d, const int* __restrict__ block_table,
                                                      int max_blocks, int q_len, T* __restrict__ kc,
                                                      T* __restrict__ vc) {
  const int t = blockIdx.x;
  const int half = d >> 1;
  const int ld = (nq + 2 * nkv) * d;
  const int p = positions[t];
  const int b = t / q_len;
  const int blk = block_table[(size_t)b * max_blocks + p / kKvBlock];
  const int row = p % kKvBlock;
  T* x = qkv + (size_t)t * ld;
  const float2* cs = table + (size_t)p * half;

  const int pairs = (nq + nkv) * half;
  for (int idx = threadIdx.x; idx < pairs; idx += blockDim.x) {
    const int head = idx / half;
    const int i = idx - head * half;
    const float2 c = cs[i];
    const float x0 = to_f32(x[head * d + i]);
    const float x1 = to_f32(x[head * d + i + half]);
    const float y0 = fmaf(x0, c.x, -(x1 * c.y));
    const float y1 = fmaf(x1, c.x, x0 * c.y);
    if (head < nq) {
      x[head * d + i] = from_f32<T>(y0);
      x[head * d + i + half] = from_f32<T>(y1);
    } else {
      const int gk = head - nq;
      T* dst = kc + (((size_t)blk * nkv + gk) * kKvBlock + row) * d;
      dst[i] = from_f32<T>(y0);
      dst[i + half] = from_f32<T>(y1);
    }
  }
  const T* v = x + (size_t)(nq + nkv) * d;
  for (int idx = threadIdx.x; idx < nkv * d; idx += blockDim.x) {
    const int gv = idx / d;
    const int e = idx - gv * d;
    vc[(((size_t)blk * nkv + gv) * d + e) * kKvBlock + row] = v[idx];
  }
}

}  // namespace

hipError_t launch_rope_kv(int dtype, void* qkv, int T, const int* positions, const float2* table,
                          int nq, int nkv, int d, const int* block_table, int max_blocks, int q_len,
                          void* k_cache, void* v_cache, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dtype == kBF16) {
    rope_kv_kernel<bf16><<<T, 256, 0, s>>>((bf16*)qkv, positions, table, nq, nkv, d, block_table,
                                            max_blocks, q_len, (bf16*)k_cache, (bf16*)v_cache);
  } else {
    rope_kv_kernel<float><<<T, 256, 0, s>>>((float*)qkv, positions, table, nq, nkv, d, block_table,
                                             max_blocks, q_len, (float*)k_cache, (float*)v_cache);
  }
  return hipGetLastError();
}

}  // namespace llk
