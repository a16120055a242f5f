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
// (one wave's softmax overlaps another's MFMAs).  The key loop walks 64-key
// tiles (four 16-slot cache blocks) with an online softmax in fp32 (exp2 of
// log2(e)/sqrt(d)-scaled scores; the reference max moves only when a tile's
// max exceeds it by more than 2^8), only up to the tile's last query position
// (causal tile skipping); the diagonal tiles mask key > query position.
//
// Staging: every wave copies whole cache blocks into LDS with direct
// global->LDS loads (global_load_lds_dwordx4: no registers, no LDS store
// instructions).  Such a load writes 64 consecutive 16-byte LDS slots, so the
// bank-spreading swizzles below are made by choosing which 16-byte chunk of
// the block each lane fetches.  K keeps the cache's [16 slots][D] rows, V the
// cache's [D][16 slots] block layout.
//
// With v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T : A = 16 keys x 32 d from LDS, B = the 16 queries' q from
//       registers.  Row m = 4 grp + r of 16-key slice j holds key
//       32 (j >> 1) + 8 grp + 4 (j & 1) + r, so lane (query = l % 16,
//       grp = l / 16) ends up with 8 consecutive keys, 32 mh + 8 grp .. +7,
//       of each 32-key half mh.
//   O += P V    : A = P: lane (query, grp) supplies those 8 keys as its 8
//       k-slots -- no data movement for P.  B = V: lane (component, grp)
//       reads the same 8 keys of its component, which the block layout keeps
//       side by side: one 16-byte LDS read.  P enters as two bf16 parts, its
//       rounding and the rounding of what that leaves, each multiplied by the
//       same V operand: about 16 significant bits of P instead of bf16's 8,
//       whose rounding alone moves attention outputs by up to 2e-2 of their
//       RMS.
// Keys past the tile's last query (among them any slot past the sequence's
// last written one) enter P.V with V zeroed in registers, never as what the
// cache or LDS holds there.  When few query tiles would leave CUs idle while
// each walks a long context, the keys of a tile are split into partitions of
// whole 64-key tiles (grid z), merged afterwards by the combine kernel in
// attention.hip.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kQ = 16;         // query tokens per MFMA row tile
constexpr float kLazyLog2 = 8.0f;  // reference-max slack of the online softmax, log2 units
constexpr int kKT = 64;        // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS banks: a 16-byte read (ds_read_b128) is served eight lanes at a time,
// and is conflict-free when each group of eight consecutive lanes reads
// eight distinct 16-byte columns of a 128-byte line (measured on gfx950:
// column = (byte address / 16) % 8).
//
// K tile in LDS: [64 keys][D] bf16 in 16-byte chunks; key row `key` keeps its
// chunk c in slot c ^ ksw(key).  One S^T operand read takes one chunk from
// each of the 16 keys r0 + {0..3, 8..11, 16..19, 24..27}, eight lanes from
// r0 + {0..3, 8..11} and eight from r0 + 16 + {0..3, 8..11}; ksw is distinct
// on each of those eight.
template <int D>
__device__ __forceinline__ int ksw(int key) {
  return (key & 3) | (((key >> 3) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int k_off(int key, int c) {
  return key * D + ((c ^ ksw<D>(key)) << 3);
}
// V tile in LDS: the tile's four cache blocks as the cache stores them,
// [block][D][16 slots]; the two 8-slot halves of component d trade places
// when bit 2 of d is set, so eight consecutive components' reads of one half
// hit eight distinct columns.
template <int D>
__device__ __forceinline__ int v_off(int b, int d, int h) {
  return ((b * D + d) * 2 + (h ^ ((d >> 2) & 1))) << 3;
}

// D head dim, HPW query heads per wave, QT 16-query tiles per workgroup,
// NW waves; the G heads of a KV group take G / (NW * HPW) workgroups.  With
// 4 waves a workgroup stays within 256 registers a lane, so two workgroups
// share each CU: their waves pair up on the SIMDs without a common barrier.
template <int D, int HPW, int QT, int NW>
__global__ __launch_bounds__(NW * kWave, NW == 4 ? 2 : 1) void prefill_attention_mfma(
    const bf16* __restrict__ q, int ldq, const int* __restrict__ positions, int nq, int nkv,
    const bf16* __restrict__ kc, const bf16* __restrict__ vc, const int* __restrict__ block_table,
    int max_blocks, SeqMap map, int num_qtiles, bf16* __restrict__ out, int tpp, int parts,
    float* __restrict__ partials, int* __restrict__ row_parts) {
  constexpr int U = HPW * QT;       // (head, 16-query tile) units per wave
  constexpr int KS = D / 32;        // d-steps of S^T
  constexpr int DT = D / 16;        // 16-wide d tiles of O
  constexpr int CH = D / 8;         // 16-byte chunks per K row
  constexpr int QW = kQ * QT;       // queries per workgroup
  constexpr int BPT = kKT / kKvBlock;             // cache blocks per key tile (4)
  constexpr int IPB = kKvBlock * D / 8 / kWave;   // 16-byte chunks per lane when one wave copies a block
  constexpr int BE = kKvBlock * D;                // elements of one cache block (K or V)
  // With 8 waves, each SIMD holds one wave (0..3) that runs every tile's S,
  // softmax and P.V in order, and one deferred wave (4..7) that runs the
  // previous tile's P.V first and then this tile's S and softmax: the two
  // waves' softmax phases then fall against each other's MFMAs.  The
  // deferred P.V reads the previous tile's V while the next tile's is being
  // copied in, so V has four buffers (two without deferred waves).
  constexpr bool PP = NW == 8;
  constexpr int VB = PP ? 4 : 2;
  static_assert(NW == 4 || NW == 8, "two or one cache blocks per wave and tile");
  __shared__ __attribute__((aligned(16))) bf16 sK[2][kKT * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[VB][kKT * D];

  const int G = nq / nkv;
  // Workgroup x is KV head x % nkv, head group x / nkv % HG, of query tile
  // x / nkv / HG: the heads of one query tile are consecutive, so the
  // longest tiles of every head start first (the causal lengths are
  // unequal: longest-first keeps the tail short), and with 8 KV heads each
  // XCD (workgroups go round-robin over the 8) serves one KV head, whose
  // K/V stay in that XCD's L2.
  // This workgroup's query tile: qt of sequence b, whose rows are
  // t_begin .. t_begin+qn-1.  Uniform batch: from the grid, longest tiles
  // first over all sequences; mixed batch: from the tile table (a
  // bound-sized grid; workgroups past the table's length have nothing to
  // do).
  const int HG = G / (NW * HPW);  // workgroups per (query tile, KV head)
  const int g = (int)blockIdx.x % nkv;
  const int hgi = (int)blockIdx.x / nkv % HG;  // which heads of the group
  const int wx = (int)blockIdx.x / nkv / HG;
  int b, qt, t_begin, qn;
  if (map.tiles) {
    if (wx >= *map.ntiles) return;
    const int4 e = map.tiles[wx];
    b = e.x;
    qt = e.y;
    t_begin = e.z;
    qn = e.w;
  } else {
    const int nseq = (int)gridDim.x / nkv / HG / num_qtiles;
    qt = num_qtiles - 1 - wx / nseq;
    b = wx % nseq;
    t_begin = b * map.q_len;
    qn = map.q_len;
  }
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
  if (row_parts && blockIdx.z == 0 && g == 0 && hgi == 0 && (int)threadIdx.x < nvalid) row_parts[t0 + threadIdx.x] = np;
  const int* bt = block_table + (size_t)b * max_blocks;
  const size_t head_off = (size_t)g * BE;
  const size_t blk_stride = (size_t)nkv * BE;

  const bf16x8 zero8 = {};
  // q fragments of unit uu = (head hh, query tile u): lane (query l16,
  // grp) holds components 32 s + 8 grp .. +7
  bf16x8 qf[U][KS];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int h = g * G + (hgi * NW + wave) * HPW + hh;
      const int qi = 16 * u + l16;
      const bool ok = qi < nvalid;
      const bf16* src = q + (size_t)(t0 + (ok ? qi : 0)) * ldq + (size_t)h * D + 8 * grp;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[hh * QT + u][s] = ok ? ld16<bf16x8>(src + 32 * s) : zero8;
    }

  // ---- staging: tile kt's 4 K and 4 V cache blocks; wave w copies block
  // w (K of block w for w < 4, V of block w - 4 otherwise) with 8 waves,
  // K and V of block w with 4.  Lane chunk i (0 .. IPB-1) fills LDS slot
  // 64 i + lane of the block, from the block's chunk that the swizzle puts
  // there.
  const int kblk = wave % BPT;  // the block this wave copies
  // source chunk offsets (elements) of this lane's chunks: K rows for k_src,
  // V components for v_src; with 8 waves a wave copies only K or only V, and
  // k_src holds the offsets of whichever it copies
  int k_src[IPB], v_src[IPB];
#pragma unroll
  for (int i = 0; i < IPB; ++i) {
    const int c = kWave * i + lane;
    const int row = c / CH;                      // slot of the block = key row
    const int ko = row * D + (((c % CH) ^ ksw<D>(kblk * kKvBlock + row)) << 3);
    const int d = c >> 1;                        // V: component, half
    const int vo = d * kKvBlock + (((c & 1) ^ ((d >> 2) & 1)) << 3);
    k_src[i] = (NW == 8 && wave >= BPT) ? vo : ko;
    v_src[i] = vo;
  }
  // one block of tile kt from cache plane `plane` into LDS at dst
  auto stage_block = [&](int kt, bf16* dst, const bf16* plane, const int (&off)[IPB]) {
    const int first = kt * kKT + kblk * kKvBlock;  // first key of the block
    // a block wholly past the tile's last key is not copied (its
    // block-table entry may not exist): its keys are masked in S and its V
    // is replaced by zeros in P.V
    if (first >= key_end) return;
    const int blk = __builtin_amdgcn_readfirstlane(bt[first / kKvBlock]);
    const bf16* src = plane + (size_t)blk * blk_stride + head_off;
#pragma unroll
    for (int i = 0; i < IPB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src + off[i]),
                                       (__attribute__((address_space(3))) void*)(dst + kWave * 8 * i), 16, 0, 0);
  };
  // tile kt into K buffer kb and V buffer vb
  auto stage = [&](int kt, int kb, int vb) {
    if (NW == 8) {
      const bool is_v = wave >= BPT;
      stage_block(kt, is_v ? &sV[vb][kblk * BE] : &sK[kb][kblk * BE], is_v ? vc : kc, k_src);
    } else {
      stage_block(kt, &sK[kb][kblk * BE], kc, k_src);
      stage_block(kt, &sV[vb][kblk * BE], vc, v_src);
    }
  };

  // ---- per-lane operand offsets in LDS (the same for every tile) ---------
  // S^T operand of slice j: key 32 (j >> 1) + 4 (j & 1) + kr0, chunk 4 s + grp
  // (ksw does not see bits 2 and 5 of the key, so the slice adds a constant)
  const int kr0 = 8 * (l16 >> 2) + (l16 & 3);
  int k_rd[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) k_rd[s] = k_off<D>(kr0, 4 * s + grp);
  // P.V operand of half mh: keys 32 mh + 8 grp .. +7 of component l16
  // (+16 i for d tile i)
  int v_rd[2];
#pragma unroll
  for (int mh = 0; mh < 2; ++mh) v_rd[mh] = v_off<D>(2 * mh + (grp >> 1), l16, grp & 1);

  const float sc = kLog2e / sqrtf((float)D);
  float m_run[U], l_run[U];
  f32x4 o[U][DT];
#pragma unroll
  for (int uu = 0; uu < U; ++uu) {
    m_run[uu] = -INFINITY;
    l_run[uu] = 0.f;
#pragma unroll
    for (int i = 0; i < DT; ++i) o[uu][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // S^T (raw scores) of tile kt: 4 slices of 16 keys per unit, masked where
  // keys pass a query's position (only the tiles that reach the tile's first
  // query position, or hold unwritten slots, have such keys)
  auto scores = [&](int kt, const bf16* K, f32x4 (&s4)[U][4]) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu)
#pragma unroll
      for (int j = 0; j < 4; ++j) s4[uu][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K operands read PK steps ahead of their products; step t = (s, j),
    // j fastest, so consecutive products accumulate into different tiles.
    // The scheduling barriers keep each read where it is written: left to
    // itself the compiler moves every read next to its first use and waits
    // on it there, once per operand (with the same for V below: 4 x 2048
    // attention 419 -> 375 us, 1 x 32768 20.65 -> 19.79 ms, same bits).
    constexpr int NK = 4 * KS, PK = 4;
    auto k_at = [&](int t) {
      const int s = t / 4, j = t % 4;
      return *reinterpret_cast<const bf16x8*>(&K[k_rd[s] + (32 * (j >> 1) + 4 * (j & 1)) * D]);
    };
    bf16x8 kq[PK];
#pragma unroll
    for (int t = 0; t < PK; ++t) kq[t] = k_at(t);
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      const int s = t / 4, j = t % 4;
      const bf16x8 kf = kq[t % PK];
      if (t + PK < NK) kq[t % PK] = k_at(t + PK);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int uu = 0; uu < U; ++uu) s4[uu][j] = mfma16(kf, qf[uu][s], s4[uu][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt * kKT + kKT - 1 > p0) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int pq = p0 + 16 * (uu % QT) + l16;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kt * kKT + 32 * (j >> 1) + 8 * grp + 4 * (j & 1) + r > pq) s4[uu][j][r] = -INFINITY;
      }
    }
  };
  // online softmax of one tile's scores: P for P.V (two bf16 parts: the
  // rounding of P and the rounding of the remainder), the running reference
  // max and sum, and O rescaled where the max moved
  auto softmax = [&](const f32x4 (&s4)[U][4], bf16x8 (&pa)[U][2], bf16x8 (&pl)[U][2]) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      float bm = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // pairs fold into three-input maxima
        bm = fmaxf(fmaxf(bm, s4[uu][j][0]), s4[uu][j][1]);
        bm = fmaxf(fmaxf(bm, s4[uu][j][2]), s4[uu][j][3]);
      }
      bm = row_group_max(bm);
      // The reference max m_run only has to bound the scores closely
      // enough that exp2 stays in range: softmax is unchanged by the
      // choice, as long as O and the sum share it.  It moves (and O is
      // rescaled) only when some query's tile max exceeds it by more than
      // kLazyLog2 in log2 units, so P <= 2^kLazyLog2 (exact in bf16's
      // exponent range) and most tiles skip the rescale.
      const float m_old = m_run[uu];
      const bool keep = __all(bm * sc <= m_old * sc + kLazyLog2);
      const float m_new = keep ? m_old : fmaxf(m_old, bm);
      const float ms = m_new * sc;
      // two scores at a time: one conversion rounds both to bf16 (hi), the
      // packed pair gives both back as floats by a shift and a mask, and one
      // more conversion rounds both remainders (lo)
      float ps = 0.f;
      uint32_t hw[2][4], lw[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rp = 0; rp < 2; ++rp) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s4[uu][j][2 * rp], sc, -ms));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s4[uu][j][2 * rp + 1], sc, -ms));
          const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
          const float h0 = __uint_as_float(h << 16), h1 = __uint_as_float(h & 0xffff0000u);
          hw[j >> 1][2 * (j & 1) + rp] = h;
          lw[j >> 1][2 * (j & 1) + rp] =
              __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0 - h0, p1 - h1}, bf16x2));
          ps += p0;
          ps += p1;
        }
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
        pa[uu][mh] = __builtin_bit_cast(bf16x8, (uint4){hw[mh][0], hw[mh][1], hw[mh][2], hw[mh][3]});
        pl[uu][mh] = __builtin_bit_cast(bf16x8, (uint4){lw[mh][0], lw[mh][1], lw[mh][2], lw[mh][3]});
      }
      if (keep) {
        l_run[uu] += ps;  // reference max kept: O needs no rescale
      } else {
        const float alpha = __builtin_amdgcn_exp2f((m_old - m_new) * sc);
        l_run[uu] = l_run[uu] * alpha + ps;
        float ah[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ah[r] = __shfl(alpha, 4 * grp + r, kWave);
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[uu][i][r] *= ah[r];
      }
      m_run[uu] = m_new;
    }
  };
  // O += P V of tile kt: two 32-key halves, DT d-tiles, each V operand
  // applied to both parts of P.  On the tile that reaches past key_end, the
  // V operand's keys at or past it (unwritten cache slots or blocks not
  // copied, weighted by P = 0) are zeroed in registers: 0 times whatever bits
  // they hold could be NaN.
  auto pv_tile = [&](const bf16* V, const bf16x8 (&pa)[U][2], const bf16x8 (&pl)[U][2], auto masked_c, int kt) {
    constexpr bool masked = decltype(masked_c)::value;
    // 16-bit elements kept: the first nv of this lane's 8 keys (per half)
    uint4 keepm[2];
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      keepm[mh] = uint4{~0u, ~0u, ~0u, ~0u};
      if constexpr (masked) {
        const int nv = key_end - (kt * kKT + 32 * mh + 8 * grp);
        keepm[mh].x = nv >= 2 ? ~0u : (nv == 1 ? 0xffffu : 0u);
        keepm[mh].y = nv >= 4 ? ~0u : (nv == 3 ? 0xffffu : 0u);
        keepm[mh].z = nv >= 6 ? ~0u : (nv == 5 ? 0xffffu : 0u);
        keepm[mh].w = nv >= 8 ? ~0u : (nv == 7 ? 0xffffu : 0u);
      }
    }
    // V operands read PD steps ahead of their products (see the K reads)
    constexpr int NF = 2 * DT, PD = 4;
    bf16x8 vq[PD];
#pragma unroll
    for (int t = 0; t < PD; ++t) vq[t] = *reinterpret_cast<const bf16x8*>(&V[v_rd[t / DT] + 256 * (t % DT)]);
#pragma unroll
    for (int t = 0; t < NF; ++t) {
      const int mh = t / DT, i = t % DT;
      bf16x8 vf = vq[t % PD];
      if (t + PD < NF) vq[t % PD] = *reinterpret_cast<const bf16x8*>(&V[v_rd[(t + PD) / DT] + 256 * ((t + PD) % DT)]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (masked) {
        uint4 w = __builtin_bit_cast(uint4, vf);
        w.x &= keepm[mh].x;
        w.y &= keepm[mh].y;
        w.z &= keepm[mh].z;
        w.w &= keepm[mh].w;
        vf = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        o[uu][i] = mfma16(pa[uu][mh], vf, o[uu][i]);
        o[uu][i] = mfma16(pl[uu][mh], vf, o[uu][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto pv = [&](const bf16* V, const bf16x8 (&pa)[U][2], const bf16x8 (&pl)[U][2], int kt) {
    if (kt * kKT + kKT > key_end)
      pv_tile(V, pa, pl, std::true_type(), kt);
    else
      pv_tile(V, pa, pl, std::false_type(), kt);
  };

  // Buffer indices: K kt & 1, V kt & (VB - 1).  The index a copy writes is
  // formed as an XOR of the index read in the same tile (K: kb ^ 1; V of a
  // deferred wave: (kt - 1) & 3 ^ 2 = (kt + 1) & 3), and a deferred wave
  // issues its V copy after its P.V reads: the compiler then sees that the
  // copies in flight never write what the wave still reads, and waits for
  // them only at the tile's barrier.
  // Only the range's last tile can reach past key_end, so it is peeled off
  // the loop: the loop's P.V never masks.
  stage(kt_begin, kt_begin & 1, kt_begin & (VB - 1));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int kt_last = kt_end - 1;
  if (!PP || wave < BPT) {
    for (int kt = kt_begin; kt < kt_last; ++kt) {
      const int kb = kt & 1, vb = kt & (VB - 1);
      stage(kt + 1, kb ^ 1, VB == 2 ? vb ^ 1 : (kt + 1) & (VB - 1));
      f32x4 s4[U][4];
      scores(kt, sK[kb], s4);
      bf16x8 pa[U][2], pl[U][2];
      softmax(s4, pa, pl);
      pv_tile(sV[vb], pa, pl, std::false_type(), kt);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    f32x4 s4[U][4];
    scores(kt_last, sK[kt_last & 1], s4);
    bf16x8 pa[U][2], pl[U][2];
    softmax(s4, pa, pl);
    pv(sV[kt_last & (VB - 1)], pa, pl, kt_last);
  } else {
    bf16x8 pa[U][2], pl[U][2];
    for (int kt = kt_begin; kt <= kt_last; ++kt) {
      const int kb = kt & 1, vprev = (kt - 1) & 3;
      if (kt > kt_begin) pv_tile(sV[vprev], pa, pl, std::false_type(), kt - 1);
      if (kt < kt_last) stage(kt + 1, kb ^ 1, vprev ^ 2);
      f32x4 s4[U][4];
      scores(kt, sK[kb], s4);
      softmax(s4, pa, pl);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    pv(sV[kt_last & 3], pa, pl, kt_last);
  }

  // normalise and store: lane holds O[query 16u + 4grp + r][d = 16i + l16].
  // Of a split tile, leave (reference max in log2 units, sum, unnormalised
  // O) per (query, head, partition) for the combine kernel.
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int uu = hh * QT + u;
      const int h = g * G + (hgi * NW + wave) * HPW + hh;
      const float lt = row_group_sum(l_run[uu]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = 16 * u + 4 * grp + r;
        const float lq = __shfl(lt, 4 * grp + r, kWave);
        const float mq = __shfl(m_run[uu], 4 * grp + r, kWave);
        if (qi < nvalid) {
          if (np == 1) {
            const float inv = 1.0f / lq;
            bf16* dst = out + (size_t)(t0 + qi) * nq * D + (size_t)h * D + l16;
#pragma unroll
            for (int i = 0; i < DT; ++i) dst[16 * i] = static_cast<bf16>(o[uu][i][r] * inv);
          } else {
            float* dst = partials + (((size_t)(t0 + qi) * nq + h) * parts + blockIdx.z) * (D + kPartHead);
            if (l16 == 0) {
              dst[0] = mq * sc;
              dst[1] = lq;
            }
#pragma unroll
            for (int i = 0; i < DT; ++i) dst[kPartHead + 16 * i + l16] = o[uu][i][r];
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
  const int hg = nq / nkv / (NW * HPW);
  dim3 grid(wgs * nkv * hg, 1, tpp > 0 ? parts : 1);
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
