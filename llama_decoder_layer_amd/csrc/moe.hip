// Sparse mixture-of-experts block of a Qwen3-MoE layer.
//
// What it computes: page "LLama" (hotelren.com/news/2693952), box
// "Qwen3MoeSparseMoeBlock", and page "模型库与算子层 — 代码走读"
// (vllm-learning.pages.dev), section "Fused MoE": a replicated linear router
// gives each token one logit per expert, the token keeps its top-k experts,
// each expert is a gated FFN (silu(x Wg^T) * (x Wu^T), then its down
// projection) with merged expert weights w13 [E, 2I, H] and w2 [E, H, I], and
// the token's output is the sum of its experts' outputs weighted by the gate
// probabilities: the softmax over all experts, renormalised over the kept k
// when norm_topk_prob is set.
//
// Kernels, in launch order:
//   router             logits [T, E] fp32 = x Wr^T as S fp32 partial planes:
//                      moe_router_kernel (one wave per 16 tokens x all
//                      experts x one of S K ranges) for few tokens, the
//                      tiled GEMM's split-K partials for many;
//   moe_topk_kernel    one wave per token: the S planes summed in order,
//                      softmax statistics, each expert's rank among the
//                      token's logits (ties: lower expert), the k best
//                      written in rank order, renormalisation;
//                      ids [T*k] and weights [T*k], pair p = t*k + slot;
//   moe_align_kernel   per-expert counts, the pairs grouped by expert
//                      ("sorted" positions), the active-expert list and a
//                      table of row tiles (expert, first row, rows): one
//                      workgroup for few pairs, else count / scan / scatter
//                      kernels over chunks of 4096 pairs;
//   expert GEMMs       gate_up + SiluAndMul over each expert's gathered token
//                      rows into act [P, I] (sorted order), then down with the
//                      routing weight applied before the bf16 store, scattered
//                      to part [P, H] by pair.  Few pairs per expert (decode):
//                      weight-streaming kernel over the active experts (each
//                      expert's weight read once, nontemporal loads); many
//                      (prefill): 256 x 256 MFMA tiles over the tile table;
//   moe_sum_kernel     out[t] = sum over slots of part[t*k + slot], in slot
//                      order, fp32 accumulation.
// No atomics touch the results: the order of pairs inside an expert's group
// (set by LDS atomics) changes which rows share a tile, never a row's value.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// ------------------------------------------------------------- router -----

// D[e][t] = Wr[e,:] . x[t,:]: router rows are the MFMA's A operand, token
// rows its B operand.  One wave per workgroup computes 16 tokens x all E
// experts (E/16 accumulator tiles) over one K range: grid (ceil(T/16), S).
// A lane ends with experts 16i + 4g .. +3 of token t0 + r16; the S ranges'
// partial logits [S][T][E] are summed in order by the top-k kernel.
template <int NT>  // E / 16 accumulator tiles
__global__ __launch_bounds__(64) void moe_router_kernel(const bf16* __restrict__ x, int T, int H, int kps,
                                                        const bf16* __restrict__ wr, int E,
                                                        float* __restrict__ part) {
  const int lane = threadIdx.x;
  const int r16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const int k0 = blockIdx.y * kps;
  const int t = min(t0 + r16, T - 1);
  const bf16* xa = x + (size_t)t * H + k0 + g * 8;
  const bf16* wa = wr + (size_t)r16 * H + k0 + g * 8;
  f32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // loads run one 32-wide k step ahead of the MFMAs
  bf16x8 b = ld16<bf16x8>(xa), a[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) a[i] = ld16<bf16x8>(wa + (size_t)i * 16 * H);
  for (int k = 32; k <= kps; k += 32) {
    bf16x8 bn = b, an[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) an[i] = a[i];
    if (k < kps) {
      bn = ld16<bf16x8>(xa + k);
#pragma unroll
      for (int i = 0; i < NT; ++i) an[i] = ld16<bf16x8>(wa + (size_t)i * 16 * H + k);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = mfma16(a[i], b, acc[i]);
    b = bn;
#pragma unroll
    for (int i = 0; i < NT; ++i) a[i] = an[i];
  }
  if (t0 + r16 < T) {
    float* dst = part + ((size_t)blockIdx.y * T + t0 + r16) * E + 4 * g;
#pragma unroll
    for (int i = 0; i < NT; ++i) *reinterpret_cast<f32x4*>(dst + 16 * i) = acc[i];
  }
}

// One wave per token; lane l holds experts l, l + 64, ... (EPL of them).
// The logits are first summed over the router's S partial ranges (in order)
// and stored to `logits`.  Selection by rank: each logit becomes a 64-bit
// key, its float bits mapped to an unsigned order above the complemented
// expert index, so that larger keys are larger logits and, among equal ones,
// lower experts.  Each lane counts the keys of the token above each of its
// own -- all E keys read from LDS, which broadcasts -- and an expert whose
// rank is below k writes slot `rank`.
template <int EPL>
__global__ __launch_bounds__(256) void moe_topk_kernel(const float* __restrict__ part, int S, int T, int E, int k,
                                                       int norm, float* __restrict__ logits, int* __restrict__ ids,
                                                       float* __restrict__ wts) {
  __shared__ unsigned long long sk[4][64 * EPL];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  const bool live = t < T;  // the wave's token exists (uniform)
  float v[EPL];
  unsigned long long key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = -INFINITY;
    if (live && e < E) {
      float a = part[(size_t)t * E + e];
#pragma unroll 8
      for (int sp = 1; sp < S; ++sp) a += part[((size_t)sp * T + t) * E + e];
      v[j] = a;
      logits[(size_t)t * E + e] = a;
    }
    unsigned u = __float_as_uint(v[j] + 0.f);  // -0 -> +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    key[j] = ((unsigned long long)u << 32) | (unsigned)(0xFFFFu - e);
    sk[w][e] = key[j];
  }
  __syncthreads();
  if (!live) return;
  float m = v[0];
#pragma unroll
  for (int j = 1; j < EPL; ++j) m = fmaxf(m, v[j]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + 64 * j < E) s += expf(v[j] - m);
  s = wave_sum(s);
  int rank[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) rank[j] = 0;
#pragma unroll 8
  for (int f = 0; f < E; ++f) {
    const unsigned long long kf = sk[w][f];
#pragma unroll
    for (int j = 0; j < EPL; ++j) rank[j] += kf > key[j];
  }
  float p[EPL], kept = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    p[j] = expf(v[j] - m) / s;
    if (lane + 64 * j < E && rank[j] < k) kept += p[j];
  }
  const float wsum = wave_sum(kept);
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + 64 * j < E && rank[j] < k) {
      ids[(size_t)t * k + rank[j]] = lane + 64 * j;
      wts[(size_t)t * k + rank[j]] = norm ? p[j] / wsum : p[j];
    }
}

// ---------------------------------------------------------- alignment -----

constexpr int kMaxExperts = 256;
constexpr int kAlignVec = 8;  // 16-byte id loads per thread per pass

// Exclusive scans of (pairs, tiles, active flag) over the experts, by one
// wave (lane l owns experts 4l .. 4l+3), from the per-expert counts in cnt:
// writes seg[0..E], nactive, ntiles and the LDS arrays cur (= seg), toff
// (first tile) and aidx (slot in the active list).  Called by wave 0.
__device__ void align_scan(const int* cnt, int E, int bm, int tile_cap, int* seg, int* nactive, int* ntiles,
                           int* cur, int* toff, int* aidx) {
  const int lane = threadIdx.x & 63;
  int c[4], run = 0, nt = 0, na = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    c[j] = e < E ? cnt[e] : 0;
    run += c[j];
    nt += (c[j] + bm - 1) / bm;
    na += c[j] > 0;
  }
  int ir = run, it = nt, ia = na;  // inclusive scans across lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ur = __shfl_up(ir, o, kWave), ut = __shfl_up(it, o, kWave), ua = __shfl_up(ia, o, kWave);
    if (lane >= o) {
      ir += ur;
      it += ut;
      ia += ua;
    }
  }
  run = ir - run;
  nt = it - nt;
  na = ia - na;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    if (e < E) {
      seg[e] = run;
      cur[e] = run;
      toff[e] = nt;
      aidx[e] = c[j] > 0 ? na : -1;
    }
    run += c[j];
    nt += (c[j] + bm - 1) / bm;
    na += c[j] > 0;
  }
  if (lane == 63) {
    seg[E] = run;
    *nactive = na;
    *ntiles = min(nt, tile_cap);
  }
}

// Thread e (< E): expert e's entry in the active list and its row tiles.
__device__ void align_tiles(const int* cnt, int E, int bm, const int* cur, const int* toff, const int* aidx,
                            int* active, int4* tiles, int tile_cap) {
  const int e = threadIdx.x;
  if (e >= E || cnt[e] == 0) return;
  const int c = cnt[e];
  active[aidx[e]] = e;
  for (int i = 0; i * bm < c; ++i) {
    const int idx = toff[e] + i;
    if (idx < tile_cap) tiles[idx] = make_int4(e, cur[e] + i * bm, min(bm, c - i * bm), 0);
  }
}

// Few pairs (decode): everything in one workgroup.
__global__ __launch_bounds__(1024) void moe_align_kernel(const int* __restrict__ ids, int P, int E, int bm,
                                                         int* __restrict__ seg, int* __restrict__ sorted,
                                                         int* __restrict__ active, int* __restrict__ nactive,
                                                         int4* __restrict__ tiles, int tile_cap,
                                                         int* __restrict__ ntiles) {
  __shared__ int cnt[kMaxExperts], cur[kMaxExperts], toff[kMaxExperts], aidx[kMaxExperts];
  const int tid = threadIdx.x;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  // pairs are read 16 bytes at a time, kAlignVec per thread per pass, all
  // loads of a pass in flight together (a strided loop of single loads would
  // wait out one memory latency per pair)
  auto load_pass = [&](int base, int (&v)[kAlignVec * 4]) {
#pragma unroll
    for (int j = 0; j < kAlignVec; ++j) {
      const int i = base + (j * 1024 + tid) * 4;
      if (i + 3 < P) {
        const int4 q = *reinterpret_cast<const int4*>(ids + i);
        v[4 * j] = q.x;
        v[4 * j + 1] = q.y;
        v[4 * j + 2] = q.z;
        v[4 * j + 3] = q.w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[4 * j + r] = i + r < P ? ids[i + r] : -1;
      }
    }
  };
  constexpr int kPass = 1024 * kAlignVec * 4;
  for (int base = 0; base < P; base += kPass) {
    int v[kAlignVec * 4];
    load_pass(base, v);
#pragma unroll
    for (int j = 0; j < kAlignVec * 4; ++j)
      if (v[j] >= 0) atomicAdd(&cnt[min(v[j], E - 1)], 1);
  }
  __syncthreads();
  if (tid < 64) align_scan(cnt, E, bm, tile_cap, seg, nactive, ntiles, cur, toff, aidx);
  __syncthreads();
  align_tiles(cnt, E, bm, cur, toff, aidx, active, tiles, tile_cap);
  __syncthreads();
  for (int base = 0; base < P; base += kPass) {
    int v[kAlignVec * 4];
    load_pass(base, v);
#pragma unroll
    for (int j = 0; j < kAlignVec * 4; ++j)
      if (v[j] >= 0) sorted[atomicAdd(&cur[min(v[j], E - 1)], 1)] = base + ((j >> 2) * 1024 + tid) * 4 + (j & 3);
  }
}

// Many pairs (prefill): the same grouping over chunks of kAlignChunk pairs,
// one workgroup each, so the LDS atomics spread over many CUs.  count: each
// chunk's per-expert counts -> chunk[b][e]; scan (one workgroup): totals,
// the tables, and chunk[b][e] := the first sorted position of chunk b's
// pairs of expert e; scatter: each chunk places its pairs from there.
constexpr int kAlignChunk = 4096;  // 4 pairs per thread

__device__ __forceinline__ void load4_ids(const int* ids, int P, int i, int (&v)[4]) {
  if (i + 3 < P) {
    const int4 q = *reinterpret_cast<const int4*>(ids + i);
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = i + r < P ? ids[i + r] : -1;
  }
}

__global__ __launch_bounds__(1024) void moe_count_kernel(const int* __restrict__ ids, int P, int E,
                                                         int* __restrict__ chunk) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  int v[4];
  load4_ids(ids, P, blockIdx.x * kAlignChunk + tid * 4, v);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (v[r] >= 0) atomicAdd(&cnt[min(v[r], E - 1)], 1);
  __syncthreads();
  if (tid < E) chunk[(size_t)blockIdx.x * E + tid] = cnt[tid];
}

__global__ __launch_bounds__(256) void moe_scan_kernel(int nb, int E, int bm, int* __restrict__ chunk,
                                                       int* __restrict__ seg, int* __restrict__ active,
                                                       int* __restrict__ nactive, int4* __restrict__ tiles,
                                                       int tile_cap, int* __restrict__ ntiles) {
  __shared__ int cnt[kMaxExperts], cur[kMaxExperts], toff[kMaxExperts], aidx[kMaxExperts];
  const int tid = threadIdx.x;
  if (tid < E) {
    int c = 0;
    for (int b = 0; b < nb; ++b) c += chunk[(size_t)b * E + tid];
    cnt[tid] = c;
  }
  __syncthreads();
  if (tid < 64) align_scan(cnt, E, bm, tile_cap, seg, nactive, ntiles, cur, toff, aidx);
  __syncthreads();
  align_tiles(cnt, E, bm, cur, toff, aidx, active, tiles, tile_cap);
  if (tid < E) {
    int run = cur[tid];
    for (int b = 0; b < nb; ++b) {
      const int c = chunk[(size_t)b * E + tid];
      chunk[(size_t)b * E + tid] = run;
      run += c;
    }
  }
}

__global__ __launch_bounds__(1024) void moe_scatter_kernel(const int* __restrict__ ids, int P, int E,
                                                           const int* __restrict__ chunk, int* __restrict__ sorted) {
  __shared__ int cur[kMaxExperts];
  const int tid = threadIdx.x;
  if (tid < E) cur[tid] = chunk[(size_t)blockIdx.x * E + tid];
  __syncthreads();
  const int i = blockIdx.x * kAlignChunk + tid * 4;
  int v[4];
  load4_ids(ids, P, i, v);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (v[r] >= 0) sorted[atomicAdd(&cur[min(v[r], E - 1)], 1)] = i + r;
}

// ------------------------------------------------ expert GEMM: streaming --

enum MoeEpi { kMoeGateUp = 0, kMoeDown = 1 };

// Workgroup (j, rb): active expert j, weight rows [rb * NW*NT*16, +NW*NT*16)
// of that expert, all of its pair rows in passes of 16*MT.  Gate_up: x rows
// gathered by token (pair / k) from X [T, K]; out act [P, ldo] at the sorted
// row.  Down: x rows are act's sorted rows; out part [P, ldo] at the pair's
// row, times its routing weight.
template <int MT, int NT, int KC, int NW, int EPI>
__global__ __launch_bounds__(NW * 64) void moe_stream_kernel(const bf16* __restrict__ X, int topk,
                                                             const bf16* __restrict__ W, int wrows, int K,
                                                             WStride ws, const int* __restrict__ seg,
                                                             const int* __restrict__ sorted,
                                                             const int* __restrict__ active,
                                                             const int* __restrict__ nactive,
                                                             const float* __restrict__ wts,
                                                             bf16* __restrict__ out, int ldo) {
  constexpr int SPC = KC / 32;
  constexpr int XR = MT * 16;
  constexpr int XCH = XR * KC / 8;
  constexpr int kThreads = NW * 64;
  constexpr int XPT = (XCH + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) bf16 sx[2][XR * KC];
  if ((int)blockIdx.x >= *nactive) return;
  const int e = active[blockIdx.x];
  const int r0 = seg[e], n = seg[e + 1] - r0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = (blockIdx.y * NW + wave) * NT * 16;
  const int nchunk = K / KC;
  const bf16* We = W + (size_t)e * wrows * K;

  auto xaddr = [](int row, int c) { return row * KC + ((c ^ (row & 7)) << 3); };
  const bf16x8 zero8 = {};
  const bf16* wr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wr[t] = We + (size_t)(n0 + 16 * t) * K + (size_t)r16 * ws.rs + g * 8;

  for (int c0 = 0; c0 < n; c0 += XR) {
    const int rows = min(XR, n - c0);
    // this thread's x pieces: source row pointers for the pass
    const bf16* xp[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int id = threadIdx.x + kThreads * j;
      const int row = id / (KC / 8), c = id % (KC / 8);
      xp[j] = nullptr;
      if (id < XCH && row < rows) {
        const int src = EPI == kMoeGateUp ? sorted[r0 + c0 + row] / topk : r0 + c0 + row;
        xp[j] = X + (size_t)src * K + c * 8;
      }
    }
    bf16x8 xs[XPT];
    auto xload = [&](int kc) {
#pragma unroll
      for (int j = 0; j < XPT; ++j) xs[j] = xp[j] ? ld16<bf16x8>(xp[j] + kc) : zero8;
    };
    auto xstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < XPT; ++j) {
        const int id = threadIdx.x + kThreads * j;
        const int row = id / (KC / 8), c = id % (KC / 8);
        if (id < XCH) *reinterpret_cast<bf16x8*>(&sx[buf][xaddr(row, c)]) = xs[j];
      }
    };
    bf16x8 wn[SPC][NT];
    auto wload = [&](int kc) {
#pragma unroll
      for (int s = 0; s < SPC; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) wn[s][t] = ld16_nt<bf16x8>(wr[t] + (size_t)(kc / 32 + s) * ws.ks);
    };
    f32x4 acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

    wload(0);
    xload(0);
    xstore(0);
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
      bf16x8 wc[SPC][NT];
#pragma unroll
      for (int s = 0; s < SPC; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) wc[s][t] = wn[s][t];
      if (c + 1 < nchunk) {
        wload((c + 1) * KC);
        xload((c + 1) * KC);
      }
#pragma unroll
      for (int s = 0; s < SPC; ++s) {
        bf16x8 xf[MT];
#pragma unroll
        for (int u = 0; u < MT; ++u)
          xf[u] = *reinterpret_cast<const bf16x8*>(&sx[c & 1][xaddr(16 * u + r16, s * 4 + g)]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int u = 0; u < MT; ++u) acc[t][u] = mfma16(wc[s][t], xf[u], acc[t][u]);
      }
      if (c + 1 < nchunk) xstore((c + 1) & 1);
      __syncthreads();
    }

    // lane holds features n0 + 16t + 4g + (0..3) of pass row 16u + r16
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int m = 16 * u + r16;
      if (m >= rows) continue;
      if (EPI == kMoeGateUp) {
        bf16* dst = out + (size_t)(r0 + c0 + m) * ldo;
#pragma unroll
        for (int t = 0; t < NT; t += 2) {
          const int f = ((n0 + 16 * t) >> 5) * 16 + 4 * g;
          bf16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(silu_f(acc[t][u][r]) * acc[t + 1][u][r]);
          *reinterpret_cast<bf16x4*>(dst + f) = o;
        }
      } else {
        const int p = sorted[r0 + c0 + m];
        const float wgt = wts[p];
        bf16* dst = out + (size_t)p * ldo;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          bf16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[t][u][r] * wgt);
          *reinterpret_cast<bf16x4*>(dst + n0 + 16 * t + 4 * g) = o;
        }
      }
    }
  }
}

// ---------------------------------------------------- expert GEMM: tiles --

constexpr int kTBK = 64;
constexpr int kEntriesPerChunk = 2;

// BM pair rows x BN weight rows of one expert per workgroup (an entry of the
// tile table x one weight tile), K in stages of 64 straight from global
// memory into double-buffered XOR-swizzled LDS, as the dense tiled kernel.
// Work order: chunks of kEntriesPerChunk entries x all weight tiles are
// dealt to the 8 XCDs in turn, so that the weight tiles of one entry, which
// share its gathered x rows, run together on one XCD (chunks of 1 to 8
// entries measured the same).  A partly filled tile computes all its rows
// (rows past the entry repeat its last row and are not stored): skipping
// the MFMAs of empty 16-row sub-tiles measured no faster, the kernel being
// bound by feeding LDS rather than by MFMA issue.
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void moe_tile_kernel(const bf16* __restrict__ X, int topk,
                                                                const bf16* __restrict__ W, int wrows, int K,
                                                                WStride ws, const int4* __restrict__ tiles,
                                                                const int* __restrict__ ntiles,
                                                                const int* __restrict__ sorted,
                                                                const float* __restrict__ wts,
                                                                bf16* __restrict__ out, int ldo) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int SM = TM / 16, SN = TN / 16;
  constexpr int WJ = BN / 8 / NW;
  constexpr int XJ = BM / 8 / NW;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  bf16* sW = smem;
  bf16* sX = smem + 2 * BN * kTBK;
  auto swz = [](int row, int c) { return row * kTBK + ((c ^ (row & 7)) << 3); };

  const int nn = wrows / BN;
  const int C = nn * kEntriesPerChunk;
  const int i8 = blockIdx.x >> 3;
  const int L = ((i8 / C) * 8 + (blockIdx.x & 7)) * C + i8 % C;
  const int entry = L / nn, n_t = L % nn;
  if (entry >= *ntiles) return;
  const int4 tl = tiles[entry];
  const int r0 = tl.y, rows = tl.z;
  const bf16* We = W + (size_t)tl.x * wrows * K;
  const int n0 = n_t * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int r16 = lane & 15, g = lane >> 4;
  const int prow = lane >> 3, pc = lane & 7;

  const bf16* wsrc[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int row = n0 + (j * NW + wave) * 8 + prow;
    const int ch = pc ^ (row & 7);
    wsrc[j] = We + (size_t)(row & ~15) * K + (size_t)(row & 15) * ws.rs + (size_t)(ch >> 2) * ws.ks + (ch & 3) * 8;
  }
  const size_t wstage = (size_t)(kTBK / 32) * ws.ks;
  auto issue_w = [&](int buf, int kt) {
#pragma unroll
    for (int j = 0; j < WJ; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(wsrc[j] + kt * wstage),
          (__attribute__((address_space(3))) void*)(sW + buf * BN * kTBK + (j * NW + wave) * 8 * kTBK), 16, 0, 0);
  };
  // the weights of the first stage need no pair list: on their way first
  issue_w(0, 0);
  const bf16* xsrc[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int row = (j * NW + wave) * 8 + prow;
    const int i = min(row, rows - 1);  // rows past the entry repeat its last row, never stored
    const int src = EPI == kMoeGateUp ? sorted[r0 + i] / topk : r0 + i;
    xsrc[j] = X + (size_t)src * K + ((pc ^ (row & 7)) << 3);
  }
  auto issue_x = [&](int buf, int kt) {
#pragma unroll
    for (int j = 0; j < XJ; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(xsrc[j] + kt * kTBK),
          (__attribute__((address_space(3))) void*)(sX + buf * BM * kTBK + (j * NW + wave) * 8 * kTBK), 16, 0, 0);
  };
  issue_x(0, 0);

  // down: the pair row and routing weight of each output row, fetched now so
  // that the epilogue does not wait out two dependent loads
  int prow_out[SM];
  float pwgt[SM];
#pragma unroll
  for (int j = 0; j < SM; ++j) {
    prow_out[j] = 0;
    pwgt[j] = 0.f;
    const int m = wm * TM + j * 16 + r16;
    if (EPI == kMoeDown && m < rows) {
      prow_out[j] = sorted[r0 + m];
      pwgt[j] = wts[prow_out[j]];
    }
  }

  f32x4 acc[SN][SM];
#pragma unroll
  for (int i = 0; i < SN; ++i)
#pragma unroll
    for (int j = 0; j < SM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kTBK;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      issue_w(buf ^ 1, kt + 1);
      issue_x(buf ^ 1, kt + 1);
    }
#pragma unroll
    for (int s = 0; s < kTBK / 32; ++s) {
      const int c = s * 4 + g;
      bf16x8 b[SM];
#pragma unroll
      for (int j = 0; j < SM; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&sX[buf * BM * kTBK + swz(wm * TM + j * 16 + r16, c)]);
#pragma unroll
      for (int i = 0; i < SN; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sW[buf * BN * kTBK + swz(wn * TN + i * 16 + r16, c)]);
#pragma unroll
        for (int j = 0; j < SM; ++j) acc[i][j] = mfma16(a, b[j], acc[i][j]);
      }
    }
    // the next stage's loads have landed and every wave is done with this one
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < SM; ++j) {
    const int m = wm * TM + j * 16 + r16;
    if (m >= rows) continue;
    if (EPI == kMoeGateUp) {
      bf16* dst = out + (size_t)(r0 + m) * ldo;
#pragma unroll
      for (int i = 0; i < SN; i += 2) {
        const int f = ((n0 + wn * TN + i * 16) >> 5) * 16 + 4 * g;
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(silu_f(acc[i][j][r]) * acc[i + 1][j][r]);
        *reinterpret_cast<bf16x4*>(dst + f) = o;
      }
    } else {
      const float wgt = pwgt[j];
      bf16* dst = out + (size_t)prow_out[j] * ldo;
#pragma unroll
      for (int i = 0; i < SN; ++i) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[i][j][r] * wgt);
        *reinterpret_cast<bf16x4*>(dst + n0 + wn * TN + i * 16 + 4 * g) = o;
      }
    }
  }
}

// ------------------------------------------------------------- combine ----

// out[t][n .. n+7] = bf16(sum over slots of part[t*k + slot][n .. n+7])
__global__ __launch_bounds__(256) void moe_sum_kernel(const bf16* __restrict__ part, int T, int k, int H,
                                                      bf16* __restrict__ out) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= (size_t)T * H) return;
  const size_t t = i / H;
  const int n = (int)(i % H);
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const bf16x8 v = ld16<bf16x8>(part + (t * k + j) * H + n);
#pragma unroll
    for (int r = 0; r < 8; ++r) a[r] += static_cast<float>(v[r]);
  }
  bf16x8 o;
#pragma unroll
  for (int r = 0; r < 8; ++r) o[r] = static_cast<bf16>(a[r]);
  *reinterpret_cast<bf16x8*>(out + i) = o;
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_moe_tile(const bf16* x, int topk, const bf16* w, int wrows, int K, WStride ws, const MoeRouting& r,
                           bf16* out, int ldo, hipStream_t s) {
  auto fn = moe_tile_kernel<BM, BN, WM, WN, EPI>;
  const size_t lds = (size_t)2 * (BM + BN) * kTBK * sizeof(bf16);
  // more than 64 KiB of dynamic LDS needs the function's opt-in: done once
  // per instantiation (a thread-safe function-local static)
  static const hipError_t attr =
      lds > 65536 ? hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)
                  : hipSuccess;
  if (attr != hipSuccess) return attr;
  const int nn = wrows / BN;
  const size_t C8 = (size_t)8 * nn * kEntriesPerChunk;
  const size_t work = (size_t)r.tile_cap * nn;
  const size_t grid = (work + C8 - 1) / C8 * C8;
  fn<<<(unsigned)grid, 64 * WM * WN, lds, s>>>(x, topk, w, wrows, K, ws, r.tiles, r.ntiles, r.sorted, r.wts, out,
                                               ldo);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_moe_stream(const bf16* x, int topk, const bf16* w, int wrows, int K, WStride ws,
                             const MoeRouting& r, int E, int mt, bf16* out, int ldo, hipStream_t s) {
  constexpr int NT = 2, NW = 4;
  const int rows_per_wg = 16 * NT * NW;
  if (wrows % rows_per_wg) return hipErrorInvalidValue;
  const dim3 grid(E, wrows / rows_per_wg);
  const bool kc256 = K % 256 == 0;
  if (mt == 1) {
    if (kc256)
      moe_stream_kernel<1, NT, 256, NW, EPI><<<grid, NW * 64, 0, s>>>(x, topk, w, wrows, K, ws, r.seg, r.sorted,
                                                                     r.active, r.nactive, r.wts, out, ldo);
    else
      moe_stream_kernel<1, NT, 128, NW, EPI><<<grid, NW * 64, 0, s>>>(x, topk, w, wrows, K, ws, r.seg, r.sorted,
                                                                     r.active, r.nactive, r.wts, out, ldo);
  } else {
    if (kc256)
      moe_stream_kernel<2, NT, 256, NW, EPI><<<grid, NW * 64, 0, s>>>(x, topk, w, wrows, K, ws, r.seg, r.sorted,
                                                                     r.active, r.nactive, r.wts, out, ldo);
    else
      moe_stream_kernel<2, NT, 128, NW, EPI><<<grid, NW * 64, 0, s>>>(x, topk, w, wrows, K, ws, r.seg, r.sorted,
                                                                     r.active, r.nactive, r.wts, out, ldo);
  }
  return hipGetLastError();
}

}  // namespace

bool moe_streaming(int T) { return T <= kSkinnyMaxM; }

namespace {
bool router_on_gemm(int T, int E) { return T > kSkinnyMaxM && E % 128 == 0; }
}  // namespace

int moe_router_splits(int T, int H, int E, int num_cus) {
  if (router_on_gemm(T, E)) return tile_plan(T, E, H, num_cus).splits;
  // about 1024 single-wave workgroups; each K range a multiple of 64
  const int tiles = (T + 15) / 16;
  int S = 1;
  while (S < 8 && tiles * S * 2 <= 1024 && H % (64 * S * 2) == 0) S *= 2;
  return S;
}

hipError_t launch_moe_route(const void* x, int T, int H, const void* router, int E, int topk, bool norm,
                            float* part, float* logits, int* ids, float* wts, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (E <= 0 || E > 256 || E % 16 || H % 64 || topk < 1 || topk > 64 || topk > E) return hipErrorInvalidValue;
  const int S = moe_router_splits(T, H, E, device_cu_count());
  hipError_t e = hipSuccess;
  if (router_on_gemm(T, E)) {
    e = launch_gemm_partials(x, router, T, E, H, kRowMajor, part, s);
    if (e != hipSuccess) return e;
    return launch_moe_topk(part, S, T, E, topk, norm, logits, ids, wts, s);
  }
  const dim3 grid((T + 15) / 16, S);
  const bf16* xb = (const bf16*)x;
  const bf16* wb = (const bf16*)router;
  switch (E / 16) {
#define LLK_ROUTER_CASE(NT) \
  case NT: moe_router_kernel<NT><<<grid, 64, 0, s>>>(xb, T, H, H / S, wb, E, part); break;
    LLK_ROUTER_CASE(1) LLK_ROUTER_CASE(2) LLK_ROUTER_CASE(3) LLK_ROUTER_CASE(4) LLK_ROUTER_CASE(5)
    LLK_ROUTER_CASE(6) LLK_ROUTER_CASE(7) LLK_ROUTER_CASE(8) LLK_ROUTER_CASE(9) LLK_ROUTER_CASE(10)
    LLK_ROUTER_CASE(11) LLK_ROUTER_CASE(12) LLK_ROUTER_CASE(13) LLK_ROUTER_CASE(14) LLK_ROUTER_CASE(15)
    LLK_ROUTER_CASE(16)
#undef LLK_ROUTER_CASE
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_moe_topk(part, S, T, E, topk, norm, logits, ids, wts, s);
}

hipError_t launch_moe_topk(const float* part, int S, int T, int E, int topk, bool norm, float* logits, int* ids,
                           float* wts, hipStream_t s) {
  const unsigned blocks = (unsigned)((T + 3) / 4);
  const int epl = (E + 63) / 64;
  const int nm = norm ? 1 : 0;
  switch (epl) {
    case 1: moe_topk_kernel<1><<<blocks, 256, 0, s>>>(part, S, T, E, topk, nm, logits, ids, wts); break;
    case 2: moe_topk_kernel<2><<<blocks, 256, 0, s>>>(part, S, T, E, topk, nm, logits, ids, wts); break;
    case 3: moe_topk_kernel<3><<<blocks, 256, 0, s>>>(part, S, T, E, topk, nm, logits, ids, wts); break;
    default: moe_topk_kernel<4><<<blocks, 256, 0, s>>>(part, S, T, E, topk, nm, logits, ids, wts); break;
  }
  return hipGetLastError();
}

int moe_align_chunks(int P) { return P > 2 * kAlignChunk ? (P + kAlignChunk - 1) / kAlignChunk : 0; }

hipError_t launch_moe_align(const int* ids, int P, int E, int bm, const MoeRouting& r, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  if (E <= 0 || E > kMaxExperts || bm <= 0) return hipErrorInvalidValue;
  const int nb = moe_align_chunks(P);
  if (nb == 0) {
    moe_align_kernel<<<1, 1024, 0, s>>>(ids, P, E, bm, r.seg, r.sorted, r.active, r.nactive, r.tiles, r.tile_cap,
                                        r.ntiles);
    return hipGetLastError();
  }
  if (!r.chunk) return hipErrorInvalidValue;
  moe_count_kernel<<<nb, 1024, 0, s>>>(ids, P, E, r.chunk);
  moe_scan_kernel<<<1, 256, 0, s>>>(nb, E, bm, r.chunk, r.seg, r.active, r.nactive, r.tiles, r.tile_cap, r.ntiles);
  moe_scatter_kernel<<<nb, 1024, 0, s>>>(ids, P, E, r.chunk, r.sorted);
  return hipGetLastError();
}

hipError_t launch_moe_experts(const void* x, int T, int H, int topk, const void* w13, const void* w2, int E, int I,
                              int layout, const MoeRouting& r, void* act, void* part, hipStream_t s,
                              hipEvent_t mid) {
  if (T <= 0) return hipSuccess;
  if (layout != kTiled16x32 || H % 256 || I % 128) return hipErrorInvalidValue;
  const bf16* xb = (const bf16*)x;
  bf16* ab = (bf16*)act;
  bf16* pb = (bf16*)part;
  const WStride ws13 = weight_stride(layout, H), ws2 = weight_stride(layout, I);
  hipError_t e;
  if (moe_streaming(T)) {
    // one 16-row pass covers an expert's pairs when they average <= 12
    const int mt = T * topk <= 12 * E ? 1 : 2;
    e = launch_moe_stream<kMoeGateUp>(xb, topk, (const bf16*)w13, 2 * I, H, ws13, r, E, mt, ab, I, s);
    if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
    return launch_moe_stream<kMoeDown>(ab, topk, (const bf16*)w2, H, I, ws2, r, E, mt, pb, H, s);
  }
  e = launch_moe_tile<256, 256, 2, 4, kMoeGateUp>(xb, topk, (const bf16*)w13, 2 * I, H, ws13, r, ab, I, s);
  if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
  if (e != hipSuccess) return e;
  return launch_moe_tile<256, 256, 2, 4, kMoeDown>(ab, topk, (const bf16*)w2, H, I, ws2, r, pb, H, s);
}

hipError_t launch_moe_sum(const void* part, int T, int topk, int H, void* out, hipStream_t s) {
  const size_t total = (size_t)T * H;
  if (total == 0) return hipSuccess;
  if (H % 8) return hipErrorInvalidValue;
  moe_sum_kernel<<<(unsigned)((total / 8 + 255) / 256), 256, 0, s>>>((const bf16*)part, T, topk, H, (bf16*)out);
  return hipGetLastError();
}

}  // namespace llk
