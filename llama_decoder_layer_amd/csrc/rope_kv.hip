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
// Qwen3 attention (qk_norm): before the rotation each q and k head is
// divided by the root of its mean square plus eps and multiplied by the
// q_norm / k_norm weight [head_dim], in fp32, and rounded once to the layer
// dtype, as a stored RMSNorm output.
//
// HBM-bound and tiny: one workgroup per (token, 8 heads).  q is rotated in
// place inside the qkv buffer.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

// One workgroup per (token, group of kHeads heads of the qkv row: q heads,
// then k heads, then v heads).  S > 0: the group's part of the projection
// row is first formed from S fp32 partial rows part[s][t][:] (a split-K qkv
// projection), rounded once to the layer dtype, stored into qkv and staged
// in LDS for the rotation.
constexpr int kHeads = 8;

template <typename T, int S>
__global__ __launch_bounds__(256) void rope_kv_kernel(T* __restrict__ qkv, const int* __restrict__ positions,
                                                      const float2* __restrict__ table, int nq, int nkv,
                                                      int d, const int* __restrict__ block_table,
                                                      int max_blocks, SeqMap map, T* __restrict__ kc,
                                                      T* __restrict__ vc, const float* __restrict__ part, int T_,
                                                      const T* __restrict__ qn, const T* __restrict__ kn,
                                                      float eps) {
  __shared__ float srow[kHeads * 128];
  const int t = blockIdx.x;
  const int h0 = blockIdx.y * kHeads;
  const int nh = min(kHeads, nq + 2 * nkv - h0);
  const int half = d >> 1;
  const int ld = (nq + 2 * nkv) * d;
  const int p = positions[t];
  const int b = map.seq(t);
  const int blk = block_table[(size_t)b * max_blocks + p / kKvBlock];
  const int row = p % kKvBlock;
  T* x = qkv + (size_t)t * ld;
  const float2* cs = table + (size_t)p * half;
  const int e0 = h0 * d;          // first element of this head group in the row
  const int ne = nh * d;

  if (S > 0) {
    for (int i = threadIdx.x * 4; i < ne; i += blockDim.x * 4) {
      f32x4 v[S > 0 ? S : 1];
#pragma unroll
      for (int sp = 0; sp < S; ++sp)
        v[sp] = *reinterpret_cast<const f32x4*>(part + ((size_t)sp * T_ + t) * ld + e0 + i);
      f32x4 a = v[0];
#pragma unroll
      for (int sp = 1; sp < S; ++sp)
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] += v[sp][q];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const T r = from_f32<T>(a[q]);
        x[e0 + i + q] = r;
        srow[i + q] = to_f32(r);
      }
    }
    __syncthreads();
  }
  auto val = [&](int i) -> float { return S > 0 ? srow[i - e0] : to_f32(x[i]); };

  for (int idx = threadIdx.x; idx < nh * half; idx += blockDim.x) {
    const int head = h0 + idx / half;
    const int i = idx % half;
    if (head < nq + nkv) {  // q and k heads turn
      const float2 c = cs[i];
      float x0 = val(head * d + i);
      float x1 = val(head * d + i + half);
      if (qn) {
        // the `half` lanes of one head are consecutive and aligned (a whole
        // wave for d = 128, half a wave for d = 64) and all take this branch
        float ss = x0 * x0 + x1 * x1;
        ss = half == 64 ? group_sum<64>(ss) : group_sum<32>(ss);
        const float inv = rsqrtf(ss / (float)d + eps);
        const T* wn = head < nq ? qn : kn;
        x0 = to_f32(from_f32<T>(x0 * inv * to_f32(wn[i])));
        x1 = to_f32(from_f32<T>(x1 * inv * to_f32(wn[i + half])));
      }
      const float y0 = fmaf(x0, c.x, -(x1 * c.y));
      const float y1 = fmaf(x1, c.x, x0 * c.y);
      if (head < nq) {
        x[head * d + i] = from_f32<T>(y0);
        x[head * d + i + half] = from_f32<T>(y1);
      } else {
        T* dst = kc + (((size_t)blk * nkv + (head - nq)) * kKvBlock + row) * d;
        dst[i] = from_f32<T>(y0);
        dst[i + half] = from_f32<T>(y1);
      }
    } else {  // v heads: a copy into the slot-contiguous V plane
      const int gv = head - nq - nkv;
      T* dst = vc + ((size_t)blk * nkv + gv) * d * kKvBlock + row;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = i + j * half;
        dst[(size_t)e * kKvBlock] = S > 0 ? from_f32<T>(srow[head * d + e - e0]) : x[head * d + e];
      }
    }
  }
}

// Many rows (prefill, mixed batches), bf16: workgroup (16 consecutive rows,
// y).  y < ceil((nq + nkv) / 8): q and k heads 8y .. 8y+7 of the 16 rows;
// each thread takes 8 consecutive elements of a head's first half and the
// matching 8 of its second half (16-byte loads and stores; the d/16 threads
// of a head reduce the q/k norm's sum of squares among themselves).  The
// last y: the v heads of the 16 rows, staged in LDS, then written one (row,
// component) slot per lane with the lanes ordered row-fastest, so the 16
// slots of a component -- 32 contiguous bytes of the V plane when the rows
// are consecutive positions of one block -- go out together.
constexpr int kRows = 16;
constexpr int kRowHeads = 8;

template <int D>
__global__ __launch_bounds__(256) void rope_kv_rows_kernel(bf16* __restrict__ qkv, int T, const int* __restrict__ positions,
                                                           const float2* __restrict__ table, int nq, int nkv,
                                                           const int* __restrict__ block_table, int max_blocks,
                                                           SeqMap map, bf16* __restrict__ kc, bf16* __restrict__ vc,
                                                           const bf16* __restrict__ qn, const bf16* __restrict__ kn,
                                                           float eps) {
  constexpr int HALF = D / 2, TPH = HALF / 8;  // threads per head
  extern __shared__ __attribute__((aligned(16))) bf16 sv[];  // [kRows][nkv * D]
  const int t0 = blockIdx.x * kRows;
  const int ld = (nq + 2 * nkv) * D;
  const int vw = nkv * D;  // v elements of a row

  const int qk_groups = (nq + nkv + kRowHeads - 1) / kRowHeads;
  if ((int)blockIdx.y < qk_groups) {
    // ---- q and k heads h0 .. h0 + nh - 1 of the 16 rows
    const int h0 = blockIdx.y * kRowHeads, nh = min(kRowHeads, nq + nkv - h0);
    const int items = kRows * nh * TPH;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
      const int part = it % TPH;
      const int hr = it / TPH;
      const int head = h0 + hr % nh, r = hr / nh;
      const int t = t0 + r;
      const bool live = t < T;  // the TPH threads of a head agree
      const int tt = live ? t : T - 1;
      const int p = positions[tt];
      bf16* x = qkv + (size_t)tt * ld + head * D + 8 * part;
      const bf16x8 a = ld16<bf16x8>(x), b = ld16<bf16x8>(x + HALF);
      float x0[8], x1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x0[e] = static_cast<float>(a[e]);
        x1[e] = static_cast<float>(b[e]);
      }
      if (qn) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x0[e] * x0[e] + x1[e] * x1[e];
        ss = group_sum<TPH>(ss);
        const float inv = rsqrtf(ss / (float)D + eps);
        const bf16* wn = head < nq ? qn : kn;
        const bf16x8 w0 = ld16<bf16x8>(wn + 8 * part), w1 = ld16<bf16x8>(wn + HALF + 8 * part);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x0[e] = static_cast<float>(static_cast<bf16>(x0[e] * inv * static_cast<float>(w0[e])));
          x1[e] = static_cast<float>(static_cast<bf16>(x1[e] * inv * static_cast<float>(w1[e])));
        }
      }
      const float2* cs = table + (size_t)p * HALF + 8 * part;
      bf16x8 y0, y1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 c = cs[e];
        y0[e] = static_cast<bf16>(fmaf(x0[e], c.x, -(x1[e] * c.y)));
        y1[e] = static_cast<bf16>(fmaf(x1[e], c.x, x0[e] * c.y));
      }
      if (!live) continue;
      bf16* dst;
      if (head < nq) {
        dst = x;
      } else {
        const int b_ = map.seq(t);
        const int blk = block_table[(size_t)b_ * max_blocks + p / kKvBlock];
        dst = kc + (((size_t)blk * nkv + (head - nq)) * kKvBlock + p % kKvBlock) * D + 8 * part;
      }
      *reinterpret_cast<bf16x8*>(dst) = y0;
      *reinterpret_cast<bf16x8*>(dst + HALF) = y1;
    }
    return;
  }

  // ---- v heads: stage [kRows][nkv * D] and each row's slot in the V plane,
  // then slot-ordered writes
  __shared__ long long vslot[kRows];  // element offset of (block, head 0, component 0, slot); -1: no row
  if (threadIdx.x < kRows) {
    const int t = t0 + threadIdx.x;
    long long o = -1;
    if (t < T) {
      const int p = positions[t];
      const int blk = block_table[(size_t)map.seq(t) * max_blocks + p / kKvBlock];
      o = (long long)blk * nkv * D * kKvBlock + p % kKvBlock;
    }
    vslot[threadIdx.x] = o;
  }
  for (int c = threadIdx.x; c < kRows * vw / 8; c += blockDim.x) {
    const int r = c / (vw / 8), e8 = c % (vw / 8);
    const int t = min(t0 + r, T - 1);
    *reinterpret_cast<bf16x8*>(sv + r * vw + 8 * e8) = ld16<bf16x8>(qkv + (size_t)t * ld + (nq + nkv) * D + 8 * e8);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRows * vw; i += blockDim.x) {
    const int r = i % kRows, ce = i / kRows;  // row fastest; ce = h * D + component
    const long long o = vslot[r];
    if (o >= 0) vc[o + (long long)ce * kKvBlock] = sv[r * vw + ce];
  }
}

template <typename T, int S>
void launch_typed(T* qkv, int T_, const int* positions, const float2* table, int nq, int nkv, int d,
                  const int* block_table, int max_blocks, const SeqMap& map, T* kc, T* vc, const float* part,
                  const QkNorm& qkn, hipStream_t s) {
  dim3 grid(T_, (nq + 2 * nkv + kHeads - 1) / kHeads);
  rope_kv_kernel<T, S><<<grid, 256, 0, s>>>(qkv, positions, table, nq, nkv, d, block_table, max_blocks, map,
                                            kc, vc, part, T_, (const T*)qkn.q, (const T*)qkn.k, qkn.eps);
}

}  // namespace

hipError_t launch_rope_kv(int dtype, void* qkv, int T, const int* positions, const float2* table,
                          int nq, int nkv, int d, const int* block_table, int max_blocks, const SeqMap& map,
                          void* k_cache, void* v_cache, hipStream_t s, const float* part, int S,
                          const QkNorm& qkn) {
  if (T <= 0) return hipSuccess;
  if (qkn.q && (d != 64 && d != 128)) return hipErrorInvalidValue;
  if (dtype == kBF16) {
    bf16* x = (bf16*)qkv;
    bf16* kc = (bf16*)k_cache;
    bf16* vc = (bf16*)v_cache;
    if (!part && (d == 64 || d == 128)) {
      const dim3 grid((T + kRows - 1) / kRows, (nq + nkv + kRowHeads - 1) / kRowHeads + 1);
      const size_t lds = (size_t)kRows * nkv * d * sizeof(bf16);
      if (lds > 65536) return hipErrorInvalidValue;
      const bf16* qn = (const bf16*)qkn.q;
      const bf16* kn = (const bf16*)qkn.k;
      if (d == 128)
        rope_kv_rows_kernel<128><<<grid, 256, lds, s>>>(x, T, positions, table, nq, nkv, block_table, max_blocks, map,
                                                         kc, vc, qn, kn, qkn.eps);
      else
        rope_kv_rows_kernel<64><<<grid, 256, lds, s>>>(x, T, positions, table, nq, nkv, block_table, max_blocks, map,
                                                        kc, vc, qn, kn, qkn.eps);
      return hipGetLastError();
    }
    if (!part) launch_typed<bf16, 0>(x, T, positions, table, nq, nkv, d, block_table, max_blocks, map, kc, vc, nullptr, qkn, s);
    else if (S == 1) launch_typed<bf16, 1>(x, T, positions, table, nq, nkv, d, block_table, max_blocks, map, kc, vc, part, qkn, s);
    else if (S == 2) launch_typed<bf16, 2>(x, T, positions, table, nq, nkv, d, block_table, max_blocks, map, kc, vc, part, qkn, s);
    else if (S == 4) launch_typed<bf16, 4>(x, T, positions, table, nq, nkv, d, block_table, max_blocks, map, kc, vc, part, qkn, s);
    else if (S == 8) launch_typed<bf16, 8>(x, T, positions, table, nq, nkv, d, block_table, max_blocks, map, kc, vc, part, qkn, s);
    else return hipErrorInvalidValue;
  } else {
    if (part) return hipErrorInvalidValue;
    launch_typed<float, 0>((float*)qkv, T, positions, table, nq, nkv, d, block_table, max_blocks, map,
                           (float*)k_cache, (float*)v_cache, nullptr, qkn, s);
  }
  return hipGetLastError();
}

}  // namespace llk
