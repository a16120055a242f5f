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
// HBM-bound: every K/V byte of the context is read once (loads with the
// nontemporal hint) and serves all G query heads of its group.  One workgroup = (token, KV head, key partition;
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
//
// Decode after a split-K qkv projection (SP > 0 partial planes): the
// workgroup of (token t, KV head g) first forms what it needs of the
// projection row itself -- the G query heads of its group, its k and v head
// -- as the bf16 rounding of the SP fp32 partials summed in split order,
// applies the q/k norm when the model has one, rotates q and k (page "LLama",
// section "4 LlamaAttention": rotary_emb on q and k only; cos/sin from the
// layer's table, y0 = fmaf(x0, c, -(x1 * s)), y1 = fmaf(x1, c, x0 * s), each
// rounded once), and -- the workgroup whose key partition holds the token's
// own position -- writes k_rot and v into the token's cache slot before any
// wave reads that block ("模型库与算子层 — 代码走读", section "Attention 层":
// the new K/V are in the cache before attention reads it), and leaves q_rot,
// k and v in the qkv workspace row.  The arithmetic is the RoPE kernel's
// (rope_kv.hip), term for term, so the cache and workspace bits are the same
// as with that kernel in between; the step saves its launch.
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

// The fused projection reduce + RoPE + cache write of a decode row (SP > 0).
struct DecFuse {
  const float* part = nullptr;   // [SP][T][ld] fp32 partial planes of the qkv projection
  const float2* table = nullptr; // RoPE (cos, sin) [max_position][D/2]
  bf16* qkv = nullptr;           // [T][ld] workspace row: q_rot, k (before RoPE), v
  const bf16* qn = nullptr;      // q/k norm weights [D], or NULL
  const bf16* kn = nullptr;
  float eps = 0.f;
};

// Grid: (token * KV heads + KV head, partition).  The KV heads of a token
// are adjacent in launch order, so the workgroups that run together walk the same
// scattered cache blocks (the heads of a block are contiguous in the pool).
template <int D, int SP>
__global__ __launch_bounds__(kWaves * kWave) void decode_attention_mfma(
    const bf16* __restrict__ q, int ldq, const int* __restrict__ positions, int nq, int nkv,
    bf16* __restrict__ kc, bf16* __restrict__ vc, const int* __restrict__ block_table,
    int max_blocks, int part_len, int parts, float* __restrict__ partials,
    bf16* __restrict__ out, const int* __restrict__ dec, const int* __restrict__ ndec,
    const int* __restrict__ seq_of, int* __restrict__ row_parts, DecFuse fz, int T) {
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
    for (int s = 0; s < KS; ++s) kf[s] = ld16_nt<bf16x8>(kb + 32 * s);
#pragma unroll
    for (int i = 0; i < DT; ++i) vf[i] = ld8_nt<bf16x4>(vb + (size_t)i * 16 * kKvBlock);
  };

  int j = jb + wave;
  // with the fused RoPE, this wave's first block is fetched while the
  // projection row is formed -- unless it holds the new key, which the
  // prologue writes first
  bool pre = false;
  if constexpr (SP > 0) {
    pre = j < je && j != p / kKvBlock;
    if (pre) load(j);
    // ---- this row's q heads of group g, its k and v head: partials summed
    // in split order and rounded (the projection's stored value) ...
    __shared__ float sx[18 * D];                        // (G + 2) heads, G <= 16
    __shared__ __attribute__((aligned(16))) bf16 sq[16][D];  // q_rot of the group
    const int half = D / 2;
    const int nel = (G + 2) * D;
    const bool owner = part == p / part_len;            // the partition holding the new key
    auto col = [&](int e) {                             // element e of (q heads, k, v) -> qkv column
      const int h = e / D, c = e - h * D;
      return h < G ? (g * G + h) * D + c : (h == G ? (nq + g) * D + c : (nq + nkv + g) * D + c);
    };
    // the new key's cache block and this thread's cos/sin pairs do not
    // depend on the sums: their loads are issued first, so their latency
    // overlaps the partials' instead of following it
    // (G + 1) * D / 2 pairs, G <= 16, over the workgroup's threads
    constexpr int kRopeItems = (17 * (D / 2) + kWaves * kWave - 1) / (kWaves * kWave);
    const int blk = block_table[(size_t)b * max_blocks + p / kKvBlock];
    const float2* cs = fz.table + (size_t)p * half;
    float2 cpre[kRopeItems];
#pragma unroll
    for (int k = 0; k < kRopeItems; ++k) {
      const int idx = threadIdx.x + k * kWaves * kWave;
      cpre[k] = idx < (G + 1) * half ? cs[idx % half] : float2{0.f, 0.f};
    }
    // two 4-element items per thread in flight at once (G + 2 heads of D
    // make at most 2.25 passes of the workgroup for G <= 16)
    constexpr int kStride = kWaves * kWave * 4;
    for (int e0 = threadIdx.x * 4; e0 < nel; e0 += 2 * kStride) {
      f32x4 v[2][SP];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e4 = e0 + u * kStride;
        if (e4 < nel) {
          const int c0 = col(e4);  // 4 consecutive elements of one head
#pragma unroll
          for (int sp = 0; sp < SP; ++sp)
            v[u][sp] = *reinterpret_cast<const f32x4*>(fz.part + ((size_t)sp * T + t) * ldq + c0);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e4 = e0 + u * kStride;
        if (e4 >= nel) continue;
        f32x4 a = v[u][0];
#pragma unroll
        for (int sp = 1; sp < SP; ++sp)
#pragma unroll
          for (int k = 0; k < 4; ++k) a[k] += v[u][sp][k];
        bf16x4 r;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          r[k] = static_cast<bf16>(a[k]);
          sx[e4 + k] = static_cast<float>(r[k]);
        }
        if (owner && e4 >= G * D) *reinterpret_cast<bf16x4*>(fz.qkv + (size_t)t * ldq + col(e4)) = r;  // k, v
      }
    }
    __syncthreads();
    // ---- ... the q/k norm, RoPE of the G q heads and the k head, and the
    // new token's k_rot and v into its cache slot
    const int slot = p % kKvBlock;
#pragma unroll
    for (int k = 0; k < kRopeItems; ++k) {
      const int idx = threadIdx.x + k * kWaves * kWave;
      if (idx >= (G + 1) * half) break;
      const int h = idx / half, i = idx - h * half;  // h == G: the k head
      float x0 = sx[h * D + i], x1 = sx[h * D + i + half];
      if (fz.qn) {
        // the `half` lanes of one head are consecutive and aligned (a whole
        // wave for D = 128, half a wave for D = 64)
        float ss = x0 * x0 + x1 * x1;
        ss = half == 64 ? group_sum<64>(ss) : group_sum<32>(ss);
        const float inv = rsqrtf(ss / (float)D + fz.eps);
        const bf16* wn = h < G ? fz.qn : fz.kn;
        x0 = to_f32(static_cast<bf16>(x0 * inv * to_f32(wn[i])));
        x1 = to_f32(static_cast<bf16>(x1 * inv * to_f32(wn[i + half])));
      }
      const float2 c = cpre[k];
      const bf16 y0 = static_cast<bf16>(fmaf(x0, c.x, -(x1 * c.y)));
      const bf16 y1 = static_cast<bf16>(fmaf(x1, c.x, x0 * c.y));
      if (h < G) {
        sq[h][i] = y0;
        sq[h][i + half] = y1;
        if (owner) {
          bf16* qo = fz.qkv + (size_t)t * ldq + (size_t)(g * G + h) * D;
          qo[i] = y0;
          qo[i + half] = y1;
        }
      } else if (owner) {
        bf16* dst = kc + (((size_t)blk * nkv + g) * kKvBlock + slot) * D;
        dst[i] = y0;
        dst[i + half] = y1;
      }
    }
    if (owner) {  // v: a copy into the slot-contiguous V plane
      bf16* dst = vc + ((size_t)blk * nkv + g) * D * kKvBlock + slot;
      for (int e = threadIdx.x; e < D; e += kWaves * kWave)
        dst[(size_t)e * kKvBlock] = static_cast<bf16>(sx[(G + 1) * D + e]);
    }
    __syncthreads();  // the slot is written before any wave loads its block
    const bool hv = l16 < G;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = hv ? *reinterpret_cast<const bf16x8*>(&sq[l16][8 * grp + 32 * s]) : zero8;
  } else {
    const bool hv = l16 < G;
    const bf16* qrow = q + (size_t)t * ldq + (size_t)(g * G + (hv ? l16 : 0)) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = hv ? ld16<bf16x8>(qrow + 32 * s) : zero8;
  }

  if (j < je && !pre) load(j);
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

template <int D, int SP>
hipError_t launch_dec(const void* q, int ldq, int T, const int* positions, int nq, int nkv, void* k_cache,
                      void* v_cache, const int* block_table, int max_blocks, int part_len, int parts, float* partials,
                      void* out, hipStream_t s, const SeqMap* map, int* row_parts, const DecFuse& fz) {
  const int rows = map ? map->dec_cap : T;
  if (rows <= 0) return hipSuccess;
  dim3 grid(rows * nkv, parts);
  decode_attention_mfma<D, SP><<<grid, kWaves * kWave, 0, s>>>(
      (const bf16*)q, ldq, positions, nq, nkv, (bf16*)k_cache, (bf16*)v_cache, block_table, max_blocks, part_len,
      parts, partials, (bf16*)out, map ? map->dec : nullptr, map ? map->ndec : nullptr, map ? map->seq_of : nullptr,
      row_parts, fz, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                        int d, void* k_cache, void* v_cache, const int* block_table,
                                        int max_blocks, int part_len, int parts, float* partials,
                                        void* out, hipStream_t s, const SeqMap* map, int* row_parts,
                                        const DecodeRope* rope) {
  if (map && (!map->dec || !map->ndec || !map->seq_of || (parts > 1 && !row_parts))) return hipErrorInvalidValue;
  DecFuse fz;
  int SP = 0;
  if (rope) {
    // one (token, KV head) row per workgroup forms its own projection slice
    if (map || !rope->part || !rope->table || !rope->qkv || nq / nkv > 16) return hipErrorInvalidValue;
    if (rope->qkn.q && (d != 64 && d != 128)) return hipErrorInvalidValue;
    SP = rope->S;
    fz.part = rope->part;
    fz.table = rope->table;
    fz.qkv = (bf16*)rope->qkv;
    fz.qn = (const bf16*)rope->qkn.q;
    fz.kn = (const bf16*)rope->qkn.k;
    fz.eps = rope->qkn.eps;
  }
#define LLK_DEC(DD, SS) \
  return launch_dec<DD, SS>(q, ldq, T, positions, nq, nkv, k_cache, v_cache, block_table, max_blocks, part_len, \
                            parts, partials, out, s, map, row_parts, fz)
#define LLK_DEC_S(DD)                \
  switch (SP) {                      \
    case 0: LLK_DEC(DD, 0);          \
    case 1: LLK_DEC(DD, 1);          \
    case 2: LLK_DEC(DD, 2);          \
    case 4: LLK_DEC(DD, 4);          \
    case 8: LLK_DEC(DD, 8);          \
    default: return hipErrorInvalidValue; \
  }
  if (d == 128) { LLK_DEC_S(128) }
  LLK_DEC_S(64)
#undef LLK_DEC_S
#undef LLK_DEC
}

}  // namespace llk
