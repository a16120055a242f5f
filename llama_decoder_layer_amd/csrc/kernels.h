// Launchers of the gfx950 kernels (host functions, one family per .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace llk {

enum Dtype { kBF16 = 0, kFP32 = 1 };
enum Epi { kEpiStore = 0, kEpiAdd = 1, kEpiSiluMul = 2, kEpiPartial = 3 };

// rmsnorm.hip.  With xpart != NULL (bf16 only) the input row is the sum of
// S fp32 partial rows xpart[s][row][:] instead of x, rounded to bf16 first
// when round_part (the value a projection storing its output would pass on).
hipError_t launch_add_rmsnorm(int dtype, const void* x, const void* res, const void* w, float eps,
                              int rows, int hidden, void* normed, void* res_out, hipStream_t s,
                              const float* xpart = nullptr, int S = 0, bool round_part = false);

// Layouts of a bf16 weight [rows][K] that the GEMMs read.  Element (r, k)
// sits at (r/16)*16*K + (r%16)*rs + (k/32)*ks + k%32:
//   kRowMajor    rs = K,  ks = 32   (the plain [rows][K] matrix)
//   kTiled16x32  rs = 32, ks = 512  ([rows/16][K/32][16][32]: a 16-row strip
//                                    is one contiguous run of 1 KiB blocks)
// The layer keeps its weights tiled: a decode workgroup then streams a few
// long contiguous runs instead of hundreds of 16 KiB-strided rows, which
// needs far fewer address translations at once and makes the stream rate
// independent of where the allocation landed physically.
enum WeightLayout { kRowMajor = 0, kTiled16x32 = 1 };
struct WStride {
  int rs, ks;
};
inline WStride weight_stride(int layout, int K) { return layout == kTiled16x32 ? WStride{32, 512} : WStride{K, 32}; }

// gemm.hip: out = x W^T with an epilogue; picks the skinny (M <= 128) or the
// tiled kernel.  bf16 weights in `layout` (rows % 16 == 0 and K % 32 == 0
// for kTiled16x32); fp32 weights are row-major.
// With part (capacity part_cap bytes) a bf16 product whose tiles would leave
// CUs idle splits K (tile_plan) into fp32 partials there, then a reduce
// kernel applies the epilogue; without it the product runs unsplit.
hipError_t launch_linear(int dtype, const void* x, const void* w, int M, int N, int K, int epi,
                         void* out, hipStream_t s, int layout = kRowMajor, float* part = nullptr,
                         size_t part_cap = 0);
// Tiled-kernel plan for M > kSkinnyMaxM: bm token rows x 256 weight rows
// (bm = 256 or 192) and K unsplit or split in 2, 4 or 8, whichever a cost
// model measured on gfx950 prices lowest; 128 x 128 tiles for fewer than 256
// tokens or weight rows not a multiple of 256, K split while those tiles
// alone number fewer than the CUs.
struct TilePlan {
  int bm;
  int splits;
  size_t partial_bytes;  // fp32 partials the split needs (0 unsplit)
};
TilePlan tile_plan(int M, int wrows, int K, int num_cus);
hipError_t launch_reorder_gate_up(const void* src, int inter, int K, void* dst, hipStream_t s);
// fp32 partial products [tile_plan(M, wrows, K).splits][M][wrows] of x W^T on
// the tiled kernel (bf16 x and W, wrows % 128 == 0, K % 64 == 0), for a
// consumer that sums the planes in order.
hipError_t launch_gemm_partials(const void* x, const void* w, int M, int wrows, int K, int layout, float* out,
                                hipStream_t s);
// out [M, wrows/2] bf16 = SiluAndMul of the sum of S fp32 partial planes
// [S][M][wrows] of a re-ordered gate_up projection (split-K).
hipError_t launch_silu_reduce(const float* part, int S, int M, int wrows, void* out, hipStream_t s);
// Row-major bf16 [rows][K] -> kTiled16x32.  With inter > 0 the source is the
// merged gate_up weight [2*inter][K] and the rows are re-ordered on the way
// as launch_reorder_gate_up does (each 32-row group: 16 gate, 16 up rows).
hipError_t launch_tile_weight(const void* src, int rows, int K, int inter, void* dst, hipStream_t s);
const char* linear_kernel_name(int dtype, int M);

// gemm_skinny.hip: bf16, M <= kSkinnyMaxM.  N = output features (SiluMul: W has 2N
// rows).  kEpiPartial writes fp32 partial sums [splits][M][N].
constexpr int kSkinnyMaxM = 128;
struct SkinnyPlan {
  int mt, nt, nw, kc, splits;  // token tiles, row tiles per wave, waves, K chunk, K splits
};
SkinnyPlan skinny_plan(int M, int wrows, int K, bool allow_split, int num_cus);
int device_cu_count();
hipError_t launch_skinny(const void* x, const void* w, int M, int N, int K, int epi, const SkinnyPlan& p,
                         void* out, hipStream_t s, int layout = kRowMajor);
hipError_t launch_splitk_reduce(const float* part, int S, int M, int N, void* out, hipStream_t s);
// In-workgroup split-K (bf16, M <= 64, N % 32 == 0, at least one 32-row
// workgroup per CU, K % 512 == 0 and K <= 4096): the final rows with a plain
// store or a residual add, without partial planes.
bool skinny_wave_split_ok(int M, int N, int K, int num_cus);
hipError_t launch_skinny_wave_split(const void* x, const void* w, int M, int N, int K, int epi, void* out,
                                    hipStream_t s, int layout);

// Token rows -> sequences.  A uniform batch (query_start_loc NULL) has q_len
// consecutive rows per sequence, so row t belongs to sequence t / q_len.  A
// mixed batch (per-sequence query counts) carries seq_of[t] and, for the
// prefill attention kernel, a table of query tiles; launch_batch_map writes
// both from query_start_loc.
struct SeqMap {
  int q_len = 0;                 // rows per sequence of a uniform batch
  const int* seq_of = nullptr;   // [T] sequence of each row (mixed batch)
  const int4* tiles = nullptr;   // (sequence, tile, first row, rows) per entry
  const int* ntiles = nullptr;   // valid entries in tiles
  int tile_cap = 0;              // capacity of tiles: the prefill grid bound
  const int* dec = nullptr;      // rows of the single-row sequences (decode attention), or NULL
  const int* ndec = nullptr;     // valid entries in dec
  int dec_cap = 0;               // capacity of dec: the decode grid bound
  __device__ __forceinline__ int seq(int t) const { return seq_of ? seq_of[t] : t / q_len; }
};

// batch_map.hip.  One workgroup.  Row starts are clamped to [0, T] and rows
// that no sequence claims map to sequence 0, so a malformed query_start_loc
// gives wrong rows but no out-of-range access.  Tiles hold qw query rows;
// a sequence's tiles are listed longest (last) first.  With dec != NULL the
// sequences with exactly one query row get no tile: their rows are listed
// in dec (sequence order, *ndec of them) for the decode attention kernel.
constexpr int kMaxMappedSeqs = 4096;
hipError_t launch_batch_map(const int* query_start_loc, int B, int T, int qw, int* seq_of, int4* tiles,
                            int tile_cap, int* ntiles, int* dec, int* ndec, hipStream_t s);

// validate.hip (debug mode).  Raises flags[k] = 1 for each broken condition
// k of the call's metadata; the caller zeroes kCheckFlags ints first.
enum CheckFlag {
  kCheckRowRanges = 0,  // query_start_loc not 0 = q[0] < q[1] < ... < q[B] = T
  kCheckSeqLens,        // a seq_lens[b] outside [max(1, rows of b), max_seq_len]
  kCheckBlockIds,       // a block id of positions < seq_lens[b] outside [0, num_blocks)
  kCheckPositions,      // a position outside [0, max_pos) or not seq_lens[b] - rows + index
  kCheckFlags
};
hipError_t launch_validate_batch(const int* positions, int T, const int* block_table, int max_blocks,
                                 const int* seq_lens, const int* query_start_loc, int B, int num_blocks, int max_pos,
                                 int max_seq_len, int* flags, hipStream_t s);

// rope_kv.hip.  With part != NULL (bf16 only) the projection row is first
// formed as the bf16 rounding of the sum of S fp32 partial rows and stored
// into qkv.  A QkNorm with weights set (Qwen3) RMS-normalises each q and k
// head before the rotation.
struct QkNorm {
  const void* q = nullptr;  // [head_dim] in the layer dtype, or NULL: no norm
  const void* k = nullptr;
  float eps = 0.f;
};
hipError_t launch_rope_kv(int dtype, void* qkv, int T, const int* positions, const float2* table,
                          int nq, int nkv, int d, const int* block_table, int max_blocks, const SeqMap& map,
                          void* k_cache, void* v_cache, hipStream_t s, const float* part = nullptr,
                          int S = 0, const QkNorm& qkn = QkNorm());

// The decode attention kernel's own RoPE / KV write (attention_decode.hip):
// the qkv projection's S fp32 partial planes, the RoPE table, the qkv
// workspace row it leaves q_rot, k and v in, and the q/k norm.
struct DecodeRope {
  const float* part = nullptr;
  int S = 0;
  const float2* table = nullptr;
  void* qkv = nullptr;
  QkNorm qkn;
};

// attention.hip.  A key partition's partial result for one (row, query
// head) is a record of D + kPartHead floats: the running max (log2 units),
// the sum of exponentials, two pad floats, then the unnormalised output
// (16-byte aligned for the combine kernel's vector loads).
constexpr int kPartHead = 4;
struct AttnPlan {
  int parts;        // key partitions per query (1 = no split): partial records per row
  int part_len;     // keys per partition of the decode kernel's rows
  int tpp;          // prefill kernel: 64-key tiles per partition (0 = no split)
  size_t ws_bytes;  // fp32 partial results
};
// decode: every sequence has exactly one query row this call.  split_prefill:
// a prefill batch runs on the matrix-core prefill kernel (bf16, supported
// group size), whose long key ranges may be split.
AttnPlan attention_plan(int T, int B, int nq, int nkv, int d, bool decode, int max_seq_len, int num_cus,
                        bool split_prefill);
// row_parts: [T] ints, used when a prefill batch's keys are split
hipError_t launch_attention(int dtype, const void* q, int ldq, int T, const int* positions, int nq,
                            int nkv, int d, void* k_cache, void* v_cache,
                            const int* block_table, int max_blocks, const SeqMap& map, bool decode,
                            const AttnPlan& plan, float* partials, int* row_parts, void* out, hipStream_t s,
                            hipEvent_t mid_event, const DecodeRope* rope = nullptr);

// attention_decode.hip (bf16, one query token per row).  Without map.dec row
// t of T is sequence t and every partition leaves partials (empty ones a max
// of -inf).  With map.dec the rows are map.dec[0 .. *map.ndec) of sequences
// map.seq_of[row]; a row whose keys fit one partition is written to out
// directly, a longer one leaves partials in its first row_parts[row]
// partitions.  With rope (rows of the uniform decode batch only) the qkv
// projection arrives as S fp32 partial planes [S][T][ldq]: each workgroup
// sums and rounds its own q, k, v heads, applies the q/k norm and RoPE,
// writes the new k_rot / v into the cache slot and q_rot, k, v into the qkv
// row (`q` is then not read) -- the work of launch_rope_kv with partials.
hipError_t launch_decode_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                        int d, void* k_cache, void* v_cache, const int* block_table,
                                        int max_blocks, int part_len, int parts, float* partials,
                                        void* out, hipStream_t s, const SeqMap* map = nullptr,
                                        int* row_parts = nullptr, const DecodeRope* rope = nullptr);

// attention_prefill.hip (bf16, G in {4, 8, 16}).  A uniform batch launches
// one workgroup per (sequence, query tile, KV head); a mixed batch one per
// entry of map.tiles, whose tiles must hold prefill_tile_rows() rows.  With
// tpp > 0 each query tile's keys are split into partitions of tpp 64-key
// tiles (grid z = parts): a tile with one partition is written to out, a
// longer one leaves partials and records its partition count in row_parts.
bool prefill_attention_supported(int nq, int nkv, int d);
int prefill_tile_rows(int nq, int nkv, int d);
hipError_t launch_prefill_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                         int d, const void* k_cache, const void* v_cache, const int* block_table,
                                         int max_blocks, const SeqMap& map, void* out, hipStream_t s, int tpp = 0,
                                         int parts = 1, float* partials = nullptr, int* row_parts = nullptr);

// moe.hip: the sparse MoE block (bf16).  Pair p = t * topk + slot.
// launch_moe_route: logits [T, E] fp32, ids and wts [T * topk] (E % 16 == 0,
// E <= 256, H % 64 == 0, topk <= min(E, 64)); part holds the router's
// moe_router_splits(T, H) partial logit planes [S][T][E].  launch_moe_align groups the
// pairs by expert (one workgroup) into the routing tables below, with tiles of
// at most bm pair rows.  launch_moe_experts: act [P, I] (sorted rows) and part
// [P, H] (pair rows, weighted) from the expert weights w13 [E][2I][H] (each
// expert's gate_up re-ordered, 16 gate + 16 up rows per 32) and w2 [E][H][I],
// both kTiled16x32; H % 256 == 0, I % 128 == 0.  launch_moe_sum: out [T, H]
// = sum over slots of part, in slot order.
constexpr int kMoeTileRows = 256;
struct MoeRouting {
  int* seg = nullptr;       // [E + 1] first sorted position of each expert
  int* sorted = nullptr;    // [P] pair of each sorted position
  int* active = nullptr;    // [E] experts with pairs, ascending
  int* nactive = nullptr;   // [1]
  int4* tiles = nullptr;    // [tile_cap] (expert, first sorted row, rows, 0)
  int* ntiles = nullptr;    // [1]
  int tile_cap = 0;         // >= P / bm + E
  float* wts = nullptr;     // [P] routing weight of each pair
  int* chunk = nullptr;     // [moe_align_chunks(P)][E] grouping scratch (many pairs)
};
int moe_align_chunks(int P);  // 0: the grouping runs in one workgroup
bool moe_streaming(int T);
// K ranges of the router: many tokens with E % 128 == 0 run the router on the
// tiled GEMM (its split-K plan), otherwise on moe_router_kernel
int moe_router_splits(int T, int H, int E, int num_cus);
hipError_t launch_moe_route(const void* x, int T, int H, const void* router, int E, int topk, bool norm,
                            float* part, float* logits, int* ids, float* wts, hipStream_t s);
// top-k of each token from S partial logit planes [S][T][E] (summed in order)
hipError_t launch_moe_topk(const float* part, int S, int T, int E, int topk, bool norm, float* logits, int* ids,
                           float* wts, hipStream_t s);
hipError_t launch_moe_align(const int* ids, int P, int E, int bm, const MoeRouting& r, hipStream_t s);
hipError_t launch_moe_experts(const void* x, int T, int H, int topk, const void* w13, const void* w2, int E, int I,
                              int layout, const MoeRouting& r, void* act, void* part, hipStream_t s,
                              hipEvent_t mid = nullptr);  // recorded between the two GEMMs
hipError_t launch_moe_sum(const void* part, int T, int topk, int H, void* out, hipStream_t s);

// diag.hip: a read-only stream of `bytes` (a multiple of 16) from src, each
// of `workgroups` workgroups of `threads` threads reading one contiguous
// region with 16-byte loads; one word per thread goes to sink
// [workgroups * threads] so that the loads are not dropped.
hipError_t launch_stream_read(const void* src, size_t bytes, int workgroups, int threads, void* sink, bool nontemporal,
                              hipStream_t s);
// diag.hip: the blocks ids[0..n) of block_bytes each (64 * k, at most 16 KiB)
// from src, one 16-byte word per thread and block; one word per thread to
// sink [workgroups * block_bytes / 16].
hipError_t launch_block_read(const void* src, const int* ids, int n, int block_bytes, int workgroups, void* sink,
                             bool nontemporal, hipStream_t s);

// noalloc.hip: the device array that holds the workspace of the forward
// entry point that allocates nothing.  setup looks up a device's address
// once (that device current), at layer create; scratch returns it (NULL
// before setup or after a failed one).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch_setup(int device);
void* noalloc_scratch(int device);

}  // namespace llk
