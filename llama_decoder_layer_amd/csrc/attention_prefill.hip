// Prefill (many query tokens per sequence) causal GQA attention over the
// paged KV cache, bf16, flash-style on the matrix cores.
//
// Computes, for every new token of a sequence at position p and query head h
// of KV group g (G = heads / kv_heads query heads per group),
//     o_h = sum_{j<=p} softmax_j(q_h . k_j / sqrt(d)) v_j
// -- pages "LLama" (hotelren.com/news/2693952), section "4 LlamaAttention";
// "模型库与算子层 — 代码走读" (vllm-learning.pages.dev), section "Attention 层"
// (the new K/V are in the cache before attention reads it, through the
// block table).  The keys of a query are the sequence's cached context plus
// its own new tokens up to and including itself.
//
// One workgroup = (sequence, KV head g, 32 consecutive query tokens); its
// waves each take one query head of the group (two for G = 16), so every K/V
// tile is staged in LDS once for all G heads, and two waves share each SIMD
// (one wave's softmax overlaps another's MFMAs).  The key loop walks 64-key tiles (four
// 16-slot cache blocks) with an online softmax in fp32 (exp2 of
// log2(e)/sqrt(d)-scaled scores; the reference max moves only when a tile's
// max exceeds it by more than 2^8), only up to the tile's last query position
// (causal tile skipping); the diagonal tiles mask key > query position.
// With v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T : A = 16 keys x 32 d from LDS, B = the 16 queries' q from
//       registers.  Lane (query = l%16, grp = l/16) receives keys
//       4*grp .. 4*grp+3 of each 16-key slice.
//   O += P V    : A = P: lane (query, grp) supplies as its 8 k-slots its own
//       keys of two 16-key slices -- no data movement for P.  B = V: the LDS
//       copy of the V tile stores each component's 64 keys in the permuted
//       order that puts exactly those 8 keys side by side, so the operand is
//       one 16-byte read (XOR-swizzled rows keep the reads conflict-free).
//       P enters as two bf16 parts, its rounding and the rounding of what
//       that leaves, each multiplied by the same V operand: about 16
//       significant bits of P instead of bf16's 8, whose rounding alone moved
//       attention outputs by more than 1e-2 of their RMS.
// Keys past the sequence's last written slot are staged as zeros, never read
// from the cache.  When few query tiles would leave CUs idle while each
// walks a long context, the keys of a tile are split into partitions of
// whole 64-key tiles (grid z), merged afterwards by the combine kernel in
// attention.hip.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kQ = 16;         // query tokens per MFMA row tile
constexpr float kLazyLog2 = 8.0f;  // reference-max slack of the online softmax, log2 units
constexpr int kKT = 64;        // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// K tile in LDS: [64 keys][D] bf16, 16-byte chunks XOR-swizzled by key.
template <int D>
__device__ __forceinline__ int k_off(int key, int c) {
  constexpr int CH = D / 8;  // chunks per key row
  return key * D + ((c ^ (key & (CH - 1))) << 3);
}
// V tile in LDS: [D][64] bf16; key k = 32m + 16h + 4grp + r sits at
// position 32m + 8grp + 4h + r; 16-byte chunks XOR-swizzled by component.
__device__ __forceinline__ int v_pos(int key) {
  const int m = key >> 5, h = (key >> 4) & 1, grp = (key >> 2) & 3, r = key & 3;
  return 32 * m + 8 * grp + 4 * h + r;
}
__device__ __forceinline__ int v_off(int d, int pos) {
  return d * kKT + ((((pos >> 3) ^ (d & 7)) << 3) | (pos & 7));
}

// D head dim, HPW query heads per wave, QT 16-query tiles per workgroup,
// NW waves (NW * HPW = G heads).
template <int D, int HPW, int QT, int NW>
__global__ __launch_bounds__(NW * kWave) void prefill_attention_mfma(
    const bf16* __restrict__ q, int ldq, const int* __restrict__ positions, int nq, int nkv,
    const bf16* __restrict__ kc, const bf16* __restrict__ vc, const int* __restrict__ block_table,
    int max_blocks, SeqMap map, int num_qtiles, bf16* __restrict__ out, int tpp, int parts,
    float* __restrict__ partials, int* __restrict__ row_parts) {
  constexpr int KS = D / 32;        // d-steps of S^T
  constexpr int DT = D / 16;        // 16-wide d tiles of O
  constexpr int CH = D / 8;         // 16-byte chunks per K row
  constexpr int BCH = kKvBlock * D / 8;   // 16-byte chunks per cache block (K or V)
  constexpr int SPL = BCH / kWave;        // chunks per lane when one wave stages one block
  constexpr int QW = kQ * QT;             // queries per workgroup
  constexpr int BPT = kKT / kKvBlock;     // cache blocks per key tile (4)
  // With 8 waves, each SIMD holds one staging wave (0..3), which runs every
  // tile's S, softmax and P.V in order, and one deferred wave (4..7), which
  // runs the previous tile's P.V first and then this tile's S and softmax:
  // the two waves' softmax phases then fall against each other's MFMAs.  The
  // deferred P.V reads the previous tile's V, so V has three buffers.
  constexpr bool PP = NW == 8;
  constexpr int VB = PP ? 3 : 2;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][kKT * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[VB][D * kKT];

  const int G = nq / nkv;
  // this workgroup's query tile: qt of sequence b, whose rows are
  // t_begin .. t_begin+qn-1.  Uniform batch: from the grid, longest tiles
  // first; mixed batch: from the tile table (a bound-sized grid; workgroups
  // past the table's length have nothing to do).
  int b, qt, t_begin, qn;
  if (map.tiles) {
    if ((int)blockIdx.x >= *map.ntiles) return;
    const int4 e = map.tiles[blockIdx.x];
    b = e.x;
    qt = e.y;
    t_begin = e.z;
    qn = e.w;
  } else {
    qt = num_qtiles - 1 - (int)(blockIdx.x % num_qtiles);
    b = blockIdx.x / num_qtiles;
    t_begin = b * map.q_len;
    qn = map.q_len;
  }
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, grp = lane >> 4;

  const int t0 = t_begin + qt * QW;                         // first token row of the tile
  const int nvalid = min(QW, qn - qt * QW);                 // query rows of the tile
  const int p0 = positions[t0];                             // position of the tile's first query
  const int p_last = positions[t_begin + qn - 1];           // last written key of the sequence
  const int key_end = min(p0 + QW - 1, p_last) + 1;         // keys this tile needs
  const int ntiles = (key_end + kKT - 1) / kKT;
  // key partition z = blockIdx.z: tiles [kt_begin, kt_end).  Partitions are
  // cut only among the tiles that start at or before p0, and the last one
  // also takes the (at most one) tile after those, so every query of the
  // tile has at least one unmasked key in every partition.
  int kt_begin = 0, kt_end = ntiles, np = 1;
  if (tpp > 0) {
    const int head = p0 / kKT + 1;
    np = min((head + tpp - 1) / tpp, parts);
    const int z = blockIdx.z;
    if (z >= np) return;
    kt_begin = z * tpp;
    if (z < np - 1) kt_end = kt_begin + tpp;
  }
  if (row_parts && blockIdx.z == 0 && blockIdx.y == 0 && (int)threadIdx.x < nvalid) row_parts[t0 + threadIdx.x] = np;
  const int* bt = block_table + (size_t)b * max_blocks;
  const size_t head_off = (size_t)g * kKvBlock * D;
  const size_t blk_stride = (size_t)nkv * kKvBlock * D;

  const bf16x8 zero8 = {};
  bf16x8 qf[HPW][QT][KS];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int h = g * G + wave * HPW + hh;
      const int qi = 16 * u + l16;
      const bool ok = qi < nvalid;
      const bf16* src = q + (size_t)(t0 + (ok ? qi : 0)) * ldq + (size_t)h * D + 8 * grp;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[hh][u][s] = ok ? ld16<bf16x8>(src + 32 * s) : zero8;
    }

  // ---- staging: the 4 cache blocks of a 64-key tile, one wave per block
  // (waves 4.. of an 8-wave workgroup take no part in staging).
  // K block: 16 rows of D, chunk c = lane + 64 i -> row c / CH, chunk c % CH
  // V block: D components of 16 slots, chunk c -> component c / 2, slots
  //          8*(c%2) .. +7, stored as two 4-key pieces at permuted positions
  const bool stager = wave < BPT;
  int k_dst[SPL], v_dst[SPL][2];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int c = lane + kWave * i;
    const int key = (wave % BPT) * kKvBlock + c / CH;
    k_dst[i] = k_off<D>(key, c % CH);
    const int d = c >> 1, key0 = (wave % BPT) * kKvBlock + 8 * (c & 1);
    v_dst[i][0] = v_off(d, v_pos(key0));
    v_dst[i][1] = v_off(d, v_pos(key0 + 4));
  }
  bf16x8 kst[SPL], vst[SPL];
  auto gload = [&](int kt) {
    if (!stager) return;
    const int first = kt * kKT + wave * kKvBlock;  // first key of this wave's block
    if (first >= key_end) {
#pragma unroll
      for (int i = 0; i < SPL; ++i) kst[i] = vst[i] = zero8;
      return;
    }
    const int blk = __builtin_amdgcn_readfirstlane(bt[first / kKvBlock]);
    const bf16* kb = kc + (size_t)blk * blk_stride + head_off;
    const bf16* vb = vc + (size_t)blk * blk_stride + head_off;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      kst[i] = ld16<bf16x8>(kb + (size_t)(lane + kWave * i) * 8);
      vst[i] = ld16<bf16x8>(vb + (size_t)(lane + kWave * i) * 8);
    }
    if (first + kKvBlock > key_end) {  // the sequence's last, partly written block
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int c = lane + kWave * i;
        if (first + c / CH >= key_end) kst[i] = zero8;
        const int s0 = first + 8 * (c & 1);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (s0 + e >= key_end) vst[i][e] = static_cast<bf16>(0.f);
      }
    }
  };
  auto sstore = [&](int kt) {  // tile kt's K into sK[kt % 2], V into sV[kt % VB]
    if (!stager) return;
    const int kb = kt & 1, vb = kt % VB;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      *reinterpret_cast<bf16x8*>(&sK[kb][k_dst[i]]) = kst[i];
      bf16x4 lo, hi;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lo[r] = vst[i][r];
        hi[r] = vst[i][4 + r];
      }
      *reinterpret_cast<bf16x4*>(&sV[vb][v_dst[i][0]]) = lo;
      *reinterpret_cast<bf16x4*>(&sV[vb][v_dst[i][1]]) = hi;
    }
  };

  // ---- per-lane operand offsets in LDS (the same for every tile) ---------
  int k_rd[KS];  // key 16j + l16 (j added below), chunk 4s + grp
#pragma unroll
  for (int s = 0; s < KS; ++s) k_rd[s] = k_off<D>(l16, 4 * s + grp);
  int v_rd[2];   // component 16i + l16 (i added below), positions 32mh + 8grp
#pragma unroll
  for (int mh = 0; mh < 2; ++mh) v_rd[mh] = v_off(l16, 32 * mh + 8 * grp);

  const float sc = kLog2e / sqrtf((float)D);
  float m_run[HPW][QT], l_run[HPW][QT];
  f32x4 o[HPW][QT][DT];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      m_run[hh][u] = -INFINITY;
      l_run[hh][u] = 0.f;
#pragma unroll
      for (int i = 0; i < DT; ++i) o[hh][u][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // S^T (raw scores) of tile kt: 4 slices of 16 keys per (head, query tile),
  // masked where keys pass a query's position (only the tiles that reach the
  // tile's first query position, or hold unwritten slots, have such keys)
  auto scores = [&](int kt, f32x4 (&s4)[HPW][QT][4]) {
    const int buf = kt & 1;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int u = 0; u < QT; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) s4[hh][u][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sK[buf][k_rd[s] + 16 * D * j]);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
          for (int u = 0; u < QT; ++u) s4[hh][u][j] = mfma16(kf, qf[hh][u][s], s4[hh][u][j]);
      }
    }
    if (kt * kKT + kKT - 1 > p0) {
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        const int pq = p0 + 16 * u + l16;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (kt * kKT + 16 * j + 4 * grp + r > pq) s4[hh][u][j][r] = -INFINITY;
      }
    }
  };
  // online softmax of one tile's scores: P for P.V (two bf16 parts: the
  // rounding of P and the rounding of the remainder), the running max and
  // sum, and O rescaled where a query's max moved
  auto softmax = [&](const f32x4 (&s4)[HPW][QT][4], bf16x8 (&pa)[HPW][QT][2], bf16x8 (&pl)[HPW][QT][2]) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        float bm = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // pairs fold into three-input maxima
          bm = fmaxf(fmaxf(bm, s4[hh][u][j][0]), s4[hh][u][j][1]);
          bm = fmaxf(fmaxf(bm, s4[hh][u][j][2]), s4[hh][u][j][3]);
        }
        bm = row_group_max(bm);
        // The reference max m_run only has to bound the scores closely
        // enough that exp2 stays in range: softmax is unchanged by the
        // choice, as long as O and the sum share it.  It moves (and O is
        // rescaled) only when some query's tile max exceeds it by more than
        // kLazyLog2 in log2 units, so P <= 2^kLazyLog2 (exact in bf16's
        // exponent range) and most tiles skip the rescale.
        const float m_old = m_run[hh][u];
        const bool keep = __all(bm * sc <= m_old * sc + kLazyLog2);
        const float m_new = keep ? m_old : fmaxf(m_old, bm);
        const float ms = m_new * sc;
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pf = __builtin_amdgcn_exp2f(fmaf(s4[hh][u][j][r], sc, -ms));
            const bf16 hi = static_cast<bf16>(pf);
            pa[hh][u][j >> 1][4 * (j & 1) + r] = hi;
            pl[hh][u][j >> 1][4 * (j & 1) + r] = static_cast<bf16>(pf - static_cast<float>(hi));
            ps += pf;
          }
        if (keep) {
          l_run[hh][u] += ps;  // reference max kept: O needs no rescale
        } else {
          const float alpha = __builtin_amdgcn_exp2f((m_old - m_new) * sc);
          l_run[hh][u] = l_run[hh][u] * alpha + ps;
          float ah[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ah[r] = __shfl(alpha, 4 * grp + r, kWave);
#pragma unroll
          for (int i = 0; i < DT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[hh][u][i][r] *= ah[r];
        }
        m_run[hh][u] = m_new;
      }
  };
  // O += P V of tile kt: two 32-key halves, DT d-tiles, each V operand
  // applied to both parts of P
  auto pv = [&](int kt, const bf16x8 (&pa)[HPW][QT][2], const bf16x8 (&pl)[HPW][QT][2]) {
    const int vb = kt % VB;
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&sV[vb][v_rd[mh] + 16 * kKT * i]);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
          for (int u = 0; u < QT; ++u) {
            o[hh][u][i] = mfma16(pa[hh][u][mh], vf, o[hh][u][i]);
            o[hh][u][i] = mfma16(pl[hh][u][mh], vf, o[hh][u][i]);
          }
      }
    }
  };

  // One barrier per tile in either order.  A V buffer is rewritten (tile
  // kt + 1, during tile kt) only after the barrier that follows its last
  // reader: the deferred P.V of tile kt - 2, run during tile kt - 1.
  gload(kt_begin);
  sstore(kt_begin);
  __syncthreads();
  if (!PP || stager) {
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      if (kt + 1 < kt_end) gload(kt + 1);
      f32x4 s4[HPW][QT][4];
      scores(kt, s4);
      bf16x8 pa[HPW][QT][2], pl[HPW][QT][2];
      softmax(s4, pa, pl);
      pv(kt, pa, pl);
      if (kt + 1 < kt_end) sstore(kt + 1);
      __syncthreads();
    }
  } else {
    bf16x8 pa[HPW][QT][2], pl[HPW][QT][2];
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      if (kt > kt_begin) pv(kt - 1, pa, pl);
      f32x4 s4[HPW][QT][4];
      scores(kt, s4);
      softmax(s4, pa, pl);
      __syncthreads();
    }
    pv(kt_end - 1, pa, pl);
  }

  // normalise and store: lane holds O[query 16u + 4grp + r][d = 16i + l16].
  // Of a split tile, leave (reference max in log2 units, sum, unnormalised O) per
  // (query, head, partition) for the combine kernel.
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      float lt = l_run[hh][u];
      lt = row_group_sum(lt);
      const int h = g * G + wave * HPW + hh;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = 16 * u + 4 * grp + r;
        const float lq = __shfl(lt, 4 * grp + r, kWave);
        const float mq = __shfl(m_run[hh][u], 4 * grp + r, kWave);
        if (qi < nvalid) {
          if (np == 1) {
            const float inv = 1.0f / lq;
            bf16* dst = out + (size_t)(t0 + qi) * nq * D + (size_t)h * D + l16;
#pragma unroll
            for (int i = 0; i < DT; ++i) dst[16 * i] = static_cast<bf16>(o[hh][u][i][r] * inv);
          } else {
            float* dst = partials + (((size_t)(t0 + qi) * nq + h) * parts + blockIdx.z) * (D + kPartHead);
            if (l16 == 0) {
              dst[0] = mq * sc;
              dst[1] = lq;
            }
#pragma unroll
            for (int i = 0; i < DT; ++i) dst[kPartHead + 16 * i + l16] = o[hh][u][i][r];
          }
        }
      }
    }
}

template <int D, int HPW, int QT, int NW>
hipError_t launch_pf(const void* q, int ldq, int T, const int* positions, int nq, int nkv, const void* k_cache,
                     const void* v_cache, const int* block_table, int max_blocks, const SeqMap& map, void* out,
                     hipStream_t s, int tpp, int parts, float* partials, int* row_parts) {
  int nqt = 0, wgs;
  if (map.tiles) {
    wgs = map.tile_cap;
  } else {
    nqt = (map.q_len + kQ * QT - 1) / (kQ * QT);
    wgs = T / map.q_len * nqt;
  }
  if (wgs <= 0) return hipSuccess;
  dim3 grid(wgs, nkv, tpp > 0 ? parts : 1);
  prefill_attention_mfma<D, HPW, QT, NW><<<grid, NW * kWave, 0, s>>>(
      (const bf16*)q, ldq, positions, nq, nkv, (const bf16*)k_cache, (const bf16*)v_cache, block_table,
      max_blocks, map, nqt, (bf16*)out, tpp, parts, partials, row_parts);
  return hipGetLastError();
}

// (HPW, QT, NW) per head dimension and group size: one query head per wave
// and 32 queries per workgroup where the group allows; two waves per SIMD
// overlap one wave's softmax with another's MFMAs
#define LLK_PF_CONFIGS(X)                                         \
  X(128, 4, 1, 2, 4) X(128, 8, 1, 2, 8) X(128, 16, 2, 1, 8)       \
  X(64, 4, 1, 2, 4) X(64, 8, 1, 2, 8) X(64, 16, 2, 1, 8)

}  // namespace

bool prefill_attention_supported(int nq, int nkv, int d) {
  const int G = nq / nkv;
  return (d == 64 || d == 128) && (G == 4 || G == 8 || G == 16);
}

int prefill_tile_rows(int nq, int nkv, int d) {
  const int G = nq / nkv;
#define LLK_PF_ROWS(DD, GG, HH, QQ, WW) \
  if (d == DD && G == GG) return kQ * QQ;
  LLK_PF_CONFIGS(LLK_PF_ROWS)
#undef LLK_PF_ROWS
  return 0;
}

hipError_t launch_prefill_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                         int d, const void* k_cache, const void* v_cache, const int* block_table,
                                         int max_blocks, const SeqMap& map, void* out, hipStream_t s, int tpp,
                                         int parts, float* partials, int* row_parts) {
  const int G = nq / nkv;
  if (!map.tiles && (map.q_len <= 0 || T % map.q_len != 0)) return hipErrorInvalidValue;
  if ((tpp > 0 || parts > 1) && (parts < 2 || !partials || !row_parts)) return hipErrorInvalidValue;
#define LLK_PF_CASE(DD, GG, HH, QQ, WW)                                                                      \
  if (d == DD && G == GG)                                                                                    \
    return launch_pf<DD, HH, QQ, WW>(q, ldq, T, positions, nq, nkv, k_cache, v_cache, block_table, max_blocks, \
                                     map, out, s, tpp, parts, partials, row_parts);
  LLK_PF_CONFIGS(LLK_PF_CASE)
#undef LLK_PF_CASE
  return hipErrorInvalidValue;
}

}  // namespace llk
