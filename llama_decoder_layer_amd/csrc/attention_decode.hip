// Decode attention (one new query token per sequence) over the paged KV
// cache, bf16, on the matrix cores.
//
// Computes, for query head h of KV group g (h = g*G .. g*G+G-1, G = heads /
// kv_heads) and the token's position p,
//     o_h = sum_{j<=p} softmax_j(q_h . k_j / sqrt(d)) v_j
// -- pages "LLama" (hotelren.com/news/2693952), section "4 LlamaAttention",
// and "模型库与算子层 — 代码走读" (vllm-learning.pages.dev), section
// "Attention 层" (attention through the block table).
//
// HBM-bound: every K/V byte of the context is read once and serves all G
// query heads of its group.  One workgroup = (token, KV head, key partition;
// a (token, KV head) is split only when that is needed to occupy every CU);
// its 4 waves take the partition's 16-slot blocks round-robin, each with its
// own running max and sum, and merge through LDS at the end.  Per block and
// wave, with v_mfma_f32_16x16x32_bf16:
//   S = K_blk q^T : A = the block's 16 K rows (a lane's 8-element slice is a
//       16-byte load of one K row), B = the group's query heads (padded to
//       16 with zeros).  Lane (head = l%16, grp = l/16) receives the scores
//       of keys 4*grp .. 4*grp+3.
//   O += P V      : the k index of this product runs over keys.  Each lane
//       supplies, as its 8 k-slots, its own four keys twice -- P rounded to
//       bf16 in the first four, the bf16 rounding of what that leaves in the
//       other four -- so P goes in straight from the lane that computed it,
//       and the B operand is the matching four slots of one V component (a
//       single 8-byte load from the V plane's slot-contiguous layout) taken
//       twice.  The one product thus applies P to about 16 significant bits
//       at no extra cost: a bf16 P alone (8 bits) flips the bf16 rounding of
//       about 40% of the attention outputs, and those flips reach the
//       residual stream and the MLP.
// Scores, max and sums are fp32 with exp2 on log2(e)/sqrt(d)-scaled scores.
// The running reference max moves
// only when a block's max exceeds it by more than 2^8 (so P <= 2^8), which
// spares most blocks the rescale of o and the sum; softmax is the same for
// any reference that o and the sum share.  Slots past the token's position
// (including the unwritten tail of the last block) are masked in both S and
// V, so stale or poisoned cache contents never reach the output.
// With several partitions each workgroup leaves (reference max, sum, unnormalised o)
// for the combine kernel in attention.hip.  In a mixed batch the kernel
// serves the sequences with a single query row from a list of their rows.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.0f;  // reference-max slack of the online softmax, log2 units

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Grid: (token * KV heads + KV head, partition).  The KV heads of a token
// are adjacent in launch order, so the workgroups that run together walk the same
// scattered cache blocks (the heads of a block are contiguous in the pool).
template <int D>
__global__ __launch_bounds__(kWaves * kWave) void decode_attention_mfma(
    const bf16* __restrict__ q, int ldq, const int* __restrict__ positions, int nq, int nkv,
    const bf16* __restrict__ kc, const bf16* __restrict__ vc, const int* __restrict__ block_table,
    int max_blocks, int part_len, int parts, float* __restrict__ partials,
    bf16* __restrict__ out, const int* __restrict__ dec, const int* __restrict__ ndec,
    const int* __restrict__ seq_of, int* __restrict__ row_parts) {
  constexpr int KS = D / 32;  // k-steps of S = K q^T
  constexpr int DT = D / 16;  // 16-wide output tiles of P V
  const int G = nq / nkv;
  const int g = blockIdx.x % nkv, part = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  int t, b;
  if (dec) {  // the single-row sequences of a mixed batch
    const int i = blockIdx.x / nkv;
    if (i >= *ndec) return;
    t = dec[i];
    b = seq_of[t];
  } else {    // one query row per sequence
    t = blockIdx.x / nkv;
    b = t;
  }
  const int p = positions[t];
  const int k_begin = part * part_len;
  const int k_end = min(p + 1, k_begin + part_len);

  if (k_begin >= k_end) {  // empty partition: only its max (-inf) is read
    if (!row_parts && threadIdx.x < G)
      partials[(((size_t)t * nq + g * G + threadIdx.x) * parts + part) * (D + kPartHead)] = -INFINITY;
    return;
  }
  // partitions that hold keys of this row; with row_parts a row of one
  // partition is final here and the combine skips it
  const int np = row_parts ? min(p / part_len + 1, parts) : parts;
  if (row_parts && part == 0 && g == 0 && threadIdx.x == 0) row_parts[t] = np;

  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_o[kWaves][16][D];

  const bf16x8 zero8 = {};
  const bf16x4 zero4 = {};
  bf16x8 qf[KS];
  {
    const bool hv = l16 < G;
    const bf16* qrow = q + (size_t)t * ldq + (size_t)(g * G + (hv ? l16 : 0)) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = hv ? ld16<bf16x8>(qrow + 32 * s) : zero8;
  }

  const float sc = kLog2e / sqrtf((float)D);
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int* bt = block_table + (size_t)b * max_blocks;
  const int jb = k_begin / kKvBlock, je = (k_end + kKvBlock - 1) / kKvBlock;
  const size_t head_stride = (size_t)kKvBlock * D;

  // fragments of the wave's next block: K rows (A of S), V slots (B of P.V)
  bf16x8 kf[KS];
  bf16x4 vf[DT];
  auto load = [&](int j) {
    const int blk = bt[j];
    const bf16* kb = kc + ((size_t)blk * nkv + g) * head_stride + (size_t)l16 * D + 8 * grp;
    const bf16* vb = vc + ((size_t)blk * nkv + g) * head_stride + (size_t)l16 * kKvBlock + 4 * grp;
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = ld16<bf16x8>(kb + 32 * s);
#pragma unroll
    for (int i = 0; i < DT; ++i) vf[i] = *reinterpret_cast<const bf16x4*>(vb + (size_t)i * 16 * kKvBlock);
  };

  int j = jb + wave;
  if (j < je) load(j);
  for (; j < je; j += kWaves) {
    bf16x8 kcur[KS];
    bf16x4 vcur[DT];
#pragma unroll
    for (int s = 0; s < KS; ++s) kcur[s] = kf[s];
#pragma unroll
    for (int i = 0; i < DT; ++i) vcur[i] = vf[i];
    if (j + kWaves < je) load(j + kWaves);

    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) sacc = mfma16(kcur[s], qf[s], sacc);

    bool valid[4];
    float sv[4];
    float bm = -INFINITY;
    const int key0 = j * kKvBlock + 4 * grp;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      valid[r] = (key0 + r >= k_begin) && (key0 + r < k_end);
      sv[r] = valid[r] ? sacc[r] * sc : -INFINITY;
      bm = fmaxf(bm, sv[r]);
    }
    // (shuffles through LDS: v_permlane swaps measured slower here, 796 ->
    // 813 us of attention on a ragged 64-sequence batch)
    bm = fmaxf(bm, __shfl_xor(bm, 16, kWave));
    bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
    // The reference max m_run moves (and o and the sum are rescaled) only
    // when some head's block max exceeds it by more than kLazyLog2 (log2
    // units): softmax does not depend on the reference, P stays <= 2^8, and
    // most blocks skip the rescale.  The first block always moves it from
    // -inf (alpha = 0).
    const bool keep = __all(bm <= m_run + kLazyLog2);
    const float m_new = keep ? m_run : fmaxf(m_run, bm);
    float ps = 0.f;
    bf16x8 pa;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = __builtin_amdgcn_exp2f(sv[r] - m_new);
      ps += pv;
      const bf16 hi = static_cast<bf16>(pv);
      pa[r] = hi;
      pa[r + 4] = static_cast<bf16>(pv - static_cast<float>(hi));  // exact difference, then rounded
    }
    if (keep) {
      l_run += ps;
    } else {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run = l_run * alpha + ps;
      // this lane's P.V output rows are heads 4*grp + r
      float ah[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ah[r] = __shfl(alpha, 4 * grp + r, kWave);
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[i][r] *= ah[r];
    }
    m_run = m_new;

#pragma unroll
    for (int i = 0; i < DT; ++i) {
      bf16x8 vb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16 v = valid[r] ? vcur[i][r] : static_cast<bf16>(0.f);
        vb[r] = v;
        vb[r + 4] = v;
      }
      o[i] = mfma16(pa, vb, o[i]);
    }
  }

  // merge the waves (a wave without blocks has m = -inf, l = 0, o = 0)
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (grp == 0) {
    s_m[wave][l16] = m_run;
    s_l[wave][l16] = l_run;
  }
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[wave][4 * grp + r][16 * i + l16] = o[i][r];
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kWaves * kWave) {
    const int h = idx / D, e = idx - (idx / D) * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][h];
      if (mw == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(mw - M);
      L = fmaf(s_l[w][h], f, L);
      O = fmaf(s_o[w][h][e], f, O);
    }
    const int qh = g * G + h;
    if (np == 1) {
      out[(size_t)t * nq * D + (size_t)qh * D + e] = static_cast<bf16>(O / L);
    } else {
      float* dst = partials + (((size_t)t * nq + qh) * parts + part) * (D + kPartHead);
      if (e == 0) {
        dst[0] = M;
        dst[1] = L;
      }
      dst[kPartHead + e] = O;
    }
  }
}

template <int D>
hipError_t launch_dec(const void* q, int ldq, int T, const int* positions, int nq, int nkv, const void* k_cache,
                      const void* v_cache, const int* block_table, int max_blocks, int part_len,
                      int parts, float* partials, void* out, hipStream_t s, const SeqMap* map, int* row_parts) {
  const int rows = map ? map->dec_cap : T;
  if (rows <= 0) return hipSuccess;
  dim3 grid(rows * nkv, parts);
  decode_attention_mfma<D><<<grid, kWaves * kWave, 0, s>>>(
      (const bf16*)q, ldq, positions, nq, nkv, (const bf16*)k_cache, (const bf16*)v_cache, block_table,
      max_blocks, part_len, parts, partials, (bf16*)out, map ? map->dec : nullptr, map ? map->ndec : nullptr,
      map ? map->seq_of : nullptr, row_parts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                        int d, const void* k_cache, const void* v_cache, const int* block_table,
                                        int max_blocks, int part_len, int parts, float* partials,
                                        void* out, hipStream_t s, const SeqMap* map, int* row_parts) {
  if (map && (!map->dec || !map->ndec || !map->seq_of || (parts > 1 && !row_parts))) return hipErrorInvalidValue;
  if (d == 128)
    return launch_dec<128>(q, ldq, T, positions, nq, nkv, k_cache, v_cache, block_table, max_blocks,
                           part_len, parts, partials, out, s, map, row_parts);
  return launch_dec<64>(q, ldq, T, positions, nq, nkv, k_cache, v_cache, block_table, max_blocks, part_len,
                        parts, partials, out, s, map, row_parts);
}

}  // namespace llk
