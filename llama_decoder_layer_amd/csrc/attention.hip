// Causal grouped-query attention over the paged KV cache.
//
// What is computed (pages "LLama", hotelren.com/news/2693952, section
// "4 LlamaAttention", and "模型库与算子层 — 代码走读",
// vllm-learning.pages.dev, section "Attention 层": attention over the cache
// through the block table): for a query token at position p and query head h,
// with KV head g = h / (heads / kv_heads),
//     o_h = sum_{j<=p} softmax_j(q_h . k_j / sqrt(d)) v_j .
// Keys are read through block_table: 16-slot blocks of the K plane
// [blocks][kv_heads][16][d] and the V plane [blocks][kv_heads][d][16].
//
// Work split: one workgroup per (query token, KV head, key partition).  The
// workgroup serves all query heads of the group from one read of each K/V
// row.  Scores, max and sums are fp32, with exp2 on log2(e)-scaled scores and
// an online (running max) softmax across chunks of keys.  With more than one
// partition each workgroup leaves (max, sum, unnormalised o) and a combine
// kernel merges the partitions with their log-sum-exp weights, in partition
// order (deterministic).
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kThreads = 256;
constexpr int kGMax = 16;      // query heads per KV head
constexpr int kChunk = 128;    // keys per softmax chunk
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void paged_attention_kernel(
    const T* __restrict__ q, int ldq, const int* __restrict__ positions, int nq, int nkv,
    const T* __restrict__ kc, const T* __restrict__ vc, const int* __restrict__ block_table,
    int max_blocks, SeqMap map, int part_len, int parts, float* __restrict__ partials,
    T* __restrict__ out) {
  using V = typename Vec16<T>::type;
  constexpr int VN = Vec16<T>::N;
  constexpr int CPT = D / VN;            // 16-byte chunks per key row
  constexpr int TPP = kThreads / CPT;    // keys per pass
  const int G = nq / nkv;

  const int t = blockIdx.x;
  const int g = blockIdx.y;
  const int part = blockIdx.z;
  const int p = positions[t];
  const int b = map.seq(t);
  const int k_begin = part * part_len;
  const int k_end = min(p + 1, k_begin + part_len);
  const int* bt = block_table + (size_t)b * max_blocks;
  const int tid = threadIdx.x;

  __shared__ float sq[kGMax][D];
  __shared__ float ss[kGMax][kChunk];
  __shared__ float s_scale[kGMax];
  __shared__ float s_m[kGMax];
  __shared__ float s_l[kGMax];

  const int out_per_thread = (G * D + kThreads - 1) / kThreads;  // <= 8 (G<=16, D<=128)
  if (k_begin >= k_end) {  // empty partition: only its max (-inf) is read
    if (tid < G) partials[(((size_t)t * nq + g * G + tid) * parts + part) * (D + kPartHead)] = -INFINITY;
    return;
  }

  const float qscale = kLog2e / sqrtf((float)D);
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, e = i % D;
    sq[h][e] = to_f32(q[(size_t)t * ldq + (size_t)(g * G + h) * D + e]) * qscale;
  }
  if (tid < G) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  __syncthreads();

  const int c = tid % CPT;
  const int lane_key = tid / CPT;
  const size_t head_off = (size_t)g * kKvBlock * D;

  for (int c0 = k_begin; c0 < k_end; c0 += kChunk) {
    const int cn = min(kChunk, k_end - c0);
    // scores of this chunk
    for (int k0 = 0; k0 < cn; k0 += TPP) {
      const int kk = k0 + lane_key;
      float dot[kGMax];
#pragma unroll
      for (int h = 0; h < kGMax; ++h) dot[h] = 0.f;
      if (kk < cn) {
        const int pos = c0 + kk;
        const int blk = bt[pos / kKvBlock];
        const T* krow = kc + (size_t)blk * nkv * kKvBlock * D + head_off + (size_t)(pos % kKvBlock) * D;
        V kv = ld16<V>(krow + c * VN);
#pragma unroll
        for (int h = 0; h < kGMax; ++h) {
          if (h < G) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < VN; ++e) a = fmaf(sq[h][c * VN + e], to_f32(kv[e]), a);
            dot[h] = a;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kGMax; ++h) {
        if (h < G) {
          const float s = group_sum<CPT>(dot[h]);
          if (c == 0 && kk < cn) ss[h][kk] = s;
        }
      }
    }
    __syncthreads();
    // online softmax update, one wave per head
    for (int h = tid / kWave; h < G; h += kThreads / kWave) {
      const int ln = tid % kWave;
      float mx = -INFINITY;
      for (int k = ln; k < cn; k += kWave) mx = fmaxf(mx, ss[h][k]);
      mx = wave_max(mx);
      const float m_old = s_m[h];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
      for (int k = ln; k < cn; k += kWave) {
        const float e = exp2f(ss[h][k] - m_new);
        ss[h][k] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (ln == 0) {
        const float sc = exp2f(m_old - m_new);  // 0 on the first chunk
        s_scale[h] = sc;
        s_l[h] = s_l[h] * sc + sum;
        s_m[h] = m_new;
      }
    }
    __syncthreads();
    // P V
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + j * kThreads;
      if (j < out_per_thread && i < G * D) {
        const int h = i / D, e = i % D;
        float a = acc[j] * s_scale[h];
        for (int k = 0; k < cn; ++k) {
          const int pos = c0 + k;
          const int blk = bt[pos / kKvBlock];
          const T* vcol = vc + (size_t)blk * nkv * kKvBlock * D + head_off + (pos % kKvBlock);
          a = fmaf(ss[h][k], to_f32(vcol[(size_t)e * kKvBlock]), a);
        }
        acc[j] = a;
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = tid + j * kThreads;
    if (j < out_per_thread && i < G * D) {
      const int h = i / D, e = i % D;
      const int qh = g * G + h;
      if (parts == 1) {
        out[(size_t)t * nq * D + (size_t)qh * D + e] = from_f32<T>(acc[j] / s_l[h]);
      } else {
        float* dst = partials + (((size_t)t * nq + qh) * parts + part) * (D + kPartHead);
        if (e == 0) {
          dst[0] = s_m[h];
          dst[1] = s_l[h];
        }
        dst[kPartHead + e] = acc[j];
      }
    }
  }
}

// Merges the key partitions of each (row, query head) with their
// log-sum-exp weights, in partition order (deterministic).  One thread per
// VEC output components; grid (rows, ceil(heads * D / VEC / kCombineThreads)).
// The partition loops are unrolled so that their loads are in flight
// together.  With row_parts, row t has row_parts[t] partitions; a row of one
// was written by the attention kernel itself.
constexpr int kCombineThreads = 256;
constexpr int kCombineVec = 4;
template <typename T, int D, int VEC>
__global__ __launch_bounds__(kCombineThreads) void attention_combine_kernel(const float* __restrict__ partials,
                                                                            int nq, int parts,
                                                                            const int* __restrict__ row_parts,
                                                                            T* __restrict__ out) {
  constexpr int R = D + kPartHead;  // floats per partition record
  const int t = blockIdx.x;
  int np = parts;
  if (row_parts) {
    np = min(row_parts[t], parts);
    if (np <= 1) return;
  }
  const int i = blockIdx.y * kCombineThreads + threadIdx.x;
  if (i >= nq * (D / VEC)) return;
  const int h = i / (D / VEC), e = (i % (D / VEC)) * VEC;
  const float* src = partials + ((size_t)t * nq + h) * parts * R;
  float M = -INFINITY;
#pragma unroll 4
  for (int k = 0; k < np; ++k) M = fmaxf(M, src[(size_t)k * R]);
  float L = 0.f;
  float o[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) o[c] = 0.f;
#pragma unroll 4
  for (int k = 0; k < np; ++k) {
    const float* pp = src + (size_t)k * R;
    const float m = pp[0];
    if (m != -INFINITY) {  // an empty partition's other fields are not written
      const float w = exp2f(m - M);
      L = fmaf(pp[1], w, L);
      float v[VEC];
      if constexpr (VEC == 4) {
        const float4 x = *reinterpret_cast<const float4*>(pp + kPartHead + e);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      } else {
        const float2 x = *reinterpret_cast<const float2*>(pp + kPartHead + e);
        v[0] = x.x; v[1] = x.y;
      }
#pragma unroll
      for (int c = 0; c < VEC; ++c) o[c] = fmaf(v[c], w, o[c]);
    }
  }
  T* dst = out + ((size_t)t * nq + h) * D + e;
#pragma unroll
  for (int c = 0; c < VEC; ++c) dst[c] = from_f32<T>(o[c] / L);
}

template <typename T, int D>
hipError_t attention_typed(const T* q, int ldq, int T_, const int* positions, int nq, int nkv,
                           const T* kc, const T* vc, const int* block_table, int max_blocks, const SeqMap& map,
                           const AttnPlan& plan, float* partials, T* out, hipStream_t s) {
  dim3 grid(T_, nkv, plan.parts);
  paged_attention_kernel<T, D><<<grid, kThreads, 0, s>>>(q, ldq, positions, nq, nkv, kc, vc, block_table,
                                                         max_blocks, map, plan.part_len, plan.parts,
                                                         partials, out);
  return hipGetLastError();
}

template <typename T>
hipError_t combine(int d, int T_, int nq, int parts, const float* partials, const int* row_parts, void* out,
                   hipStream_t s) {
  const int per_row = (nq * d / kCombineVec + kCombineThreads - 1) / kCombineThreads;
  if (d == 128)
    attention_combine_kernel<T, 128, kCombineVec><<<dim3(T_, per_row), kCombineThreads, 0, s>>>(
        partials, nq, parts, row_parts, (T*)out);
  else
    attention_combine_kernel<T, 64, kCombineVec><<<dim3(T_, per_row), kCombineThreads, 0, s>>>(
        partials, nq, parts, row_parts, (T*)out);
  return hipGetLastError();
}

}  // namespace

namespace {

// decode rows: long-running workgroups stream best, so the keys of a (row,
// KV head) are split only as far as needed to give every compute unit a
// workgroup, and no partition is longer than kMaxDecodePart keys so that one
// long sequence in a ragged batch does not leave a single workgroup
// streaming long after the rest have finished; partitions are multiples of
// 64 keys (four waves x 16-slot blocks)
int decode_part_len(long long groups, int max_seq_len, int cus) {
  constexpr int kMaxDecodePart = 4096;
  const long long want = (cus + groups - 1) / groups;
  int len = (int)((max_seq_len + want - 1) / want);
  len = (len + 63) / 64 * 64;
  if (len > kMaxDecodePart) len = kMaxDecodePart;
  return len < 64 ? 64 : len;
}

}  // namespace

AttnPlan attention_plan(int T, int B, int nq, int nkv, int d, bool decode, int max_seq_len, int num_cus,
                        bool split_prefill) {
  AttnPlan pl;
  pl.tpp = 0;
  pl.part_len = max_seq_len;
  pl.parts = 1;
  const int cus = num_cus > 0 ? num_cus : 256;
  if (decode) {
    pl.part_len = decode_part_len((long long)T * nkv, max_seq_len, cus);
    pl.parts = (max_seq_len + pl.part_len - 1) / pl.part_len;
  } else if (split_prefill) {
    // prefill on the matrix-core kernel: one workgroup per (query tile, KV
    // head) walks the tile's whole key range, and the kernel's register use
    // lets one workgroup run per CU.  A batch whose query tiles cannot fill
    // the CUs once (a short chunk on a long context, a mixed batch) would
    // leave CUs idle while a few workgroups walk thousands of keys: its keys
    // are split into partitions of whole 64-key tiles, about two workgroups
    // per CU (two rounds balance the unequal causal lengths better than
    // one), none shorter than kMinPrefillPart keys since each split row
    // costs partials written and read back.  ceil(T / tile rows) counts the
    // query tiles as if the batch were one sequence.
    constexpr int kMinPrefillPart = 512, kMaxPrefillParts = 8;
    const int qw = prefill_tile_rows(nq, nkv, d);
    const long long tiles = (long long)((T + qw - 1) / qw) * nkv;
    if (tiles < cus) {
      long long want = (2LL * cus + tiles - 1) / tiles;
      if (want > kMaxPrefillParts) want = kMaxPrefillParts;
      int len = (int)((max_seq_len + want - 1) / want);
      len = (len + 63) / 64 * 64;
      if (len < kMinPrefillPart) len = kMinPrefillPart;
      const int parts = (max_seq_len + len - 1) / len;
      if (parts > 1) {
        pl.tpp = len / 64;
        pl.parts = parts;
        // the single-row sequences of a mixed batch (at most B) on the
        // decode kernel: the decode rule, but never more partitions than
        // the prefill tiles have (the partials hold `parts` per row)
        const int dl = decode_part_len((long long)B * nkv, max_seq_len, cus);
        pl.part_len = dl > len ? dl : len;
      }
    }
  }
  pl.ws_bytes = pl.parts > 1 ? (size_t)T * nq * pl.parts * (d + kPartHead) * sizeof(float) : 0;
  return pl;
}

hipError_t launch_attention(int dtype, const void* q, int ldq, int T, const int* positions, int nq,
                            int nkv, int d, void* k_cache, void* v_cache,
                            const int* block_table, int max_blocks, const SeqMap& map, bool decode,
                            const AttnPlan& plan, float* partials, int* row_parts, void* out, hipStream_t s,
                            hipEvent_t mid_event, const DecodeRope* rope) {
  if (T <= 0) return hipSuccess;
  if (rope && !(dtype == kBF16 && decode)) return hipErrorInvalidValue;
  hipError_t e;
  int* rp = nullptr;  // per-row partition counts for the combine
  if (dtype == kBF16 && decode) {
    // one query row per sequence: row t is sequence t
    e = launch_decode_attention_bf16(q, ldq, T, positions, nq, nkv, d, k_cache, v_cache, block_table,
                                     max_blocks, plan.part_len, plan.parts, partials, out, s, nullptr, nullptr,
                                     rope);
  } else if (dtype == kBF16 && prefill_attention_supported(nq, nkv, d)) {
    // the single-row sequences of a mixed batch on the decode kernel, the
    // query tiles on the prefill kernel; with parts > 1 both record each
    // row's partition count for the combine
    if (plan.parts > 1) {
      if (!row_parts || !partials) return hipErrorInvalidValue;
      rp = row_parts;
    }
    if (map.dec) {
      e = launch_decode_attention_bf16(q, ldq, T, positions, nq, nkv, d, k_cache, v_cache, block_table,
                                       max_blocks, plan.part_len, plan.parts, partials, out, s, &map, rp);
      if (e != hipSuccess) return e;
    }
    e = launch_prefill_attention_bf16(q, ldq, T, positions, nq, nkv, d, k_cache, v_cache, block_table, max_blocks,
                                      map, out, s, plan.tpp, plan.parts, partials, rp);
  } else if (dtype == kBF16) {
    e = d == 128 ? attention_typed<bf16, 128>((const bf16*)q, ldq, T, positions, nq, nkv, (const bf16*)k_cache,
                                              (const bf16*)v_cache, block_table, max_blocks, map, plan,
                                              partials, (bf16*)out, s)
                 : attention_typed<bf16, 64>((const bf16*)q, ldq, T, positions, nq, nkv, (const bf16*)k_cache,
                                             (const bf16*)v_cache, block_table, max_blocks, map, plan, partials,
                                             (bf16*)out, s);
  } else {
    e = d == 128 ? attention_typed<float, 128>((const float*)q, ldq, T, positions, nq, nkv,
                                               (const float*)k_cache, (const float*)v_cache, block_table,
                                               max_blocks, map, plan, partials, (float*)out, s)
                 : attention_typed<float, 64>((const float*)q, ldq, T, positions, nq, nkv, (const float*)k_cache,
                                              (const float*)v_cache, block_table, max_blocks, map, plan,
                                              partials, (float*)out, s);
  }
  if (e != hipSuccess || plan.parts == 1) return e;
  if (mid_event) {
    e = hipEventRecord(mid_event, s);
    if (e != hipSuccess) return e;
  }
  return dtype == kBF16 ? combine<bf16>(d, T, nq, plan.parts, partials, rp, out, s)
                        : combine<float>(d, T, nq, plan.parts, partials, rp, out, s);
}

}  // namespace llk
