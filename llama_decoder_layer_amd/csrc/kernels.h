// Launchers of the gfx950 kernels (host functions, one family per .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace llk {

enum Dtype { kBF16 = 0, kFP32 = 1 };
enum Epi { kEpiStore = 0, kEpiAdd = 1, kEpiSiluMul = 2, kEpiPartial = 3 };

// rmsnorm.hip.  With xpart != NULL (bf16 only) the input row is the sum of
// S fp32 partial rows xpart[s][row][:] instead of x.
hipError_t launch_add_rmsnorm(int dtype, const void* x, const void* res, const void* w, float eps,
                              int rows, int hidden, void* normed, void* res_out, hipStream_t s,
                              const float* xpart = nullptr, int S = 0);

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

// gemm.hip: out = x W^T with an epilogue; picks the skinny (M <= 64) or the
// tiled kernel.  bf16 weights in `layout` (rows % 16 == 0 and K % 32 == 0
// for kTiled16x32); fp32 weights are row-major.
hipError_t launch_linear(int dtype, const void* x, const void* w, int M, int N, int K, int epi,
                         void* out, hipStream_t s, int layout = kRowMajor);
hipError_t launch_reorder_gate_up(const void* src, int inter, int K, void* dst, hipStream_t s);
// Row-major bf16 [rows][K] -> kTiled16x32.  With inter > 0 the source is the
// merged gate_up weight [2*inter][K] and the rows are re-ordered on the way
// as launch_reorder_gate_up does (each 32-row group: 16 gate, 16 up rows).
hipError_t launch_tile_weight(const void* src, int rows, int K, int inter, void* dst, hipStream_t s);
const char* linear_kernel_name(int dtype, int M);

// gemm_skinny.hip: bf16, M <= 64.  N = output features (SiluMul: W has 2N
// rows).  kEpiPartial writes fp32 partial sums [splits][M][N].
struct SkinnyPlan {
  int mt, nt, nw, kc, splits;  // token tiles, row tiles per wave, waves, K chunk, K splits
};
SkinnyPlan skinny_plan(int M, int wrows, int K, bool allow_split, int num_cus);
int device_cu_count();
hipError_t launch_skinny(const void* x, const void* w, int M, int N, int K, int epi, const SkinnyPlan& p,
                         void* out, hipStream_t s, int layout = kRowMajor);
hipError_t launch_splitk_reduce(const float* part, int S, int M, int N, void* out, hipStream_t s);

// rope_kv.hip.  With part != NULL (bf16 only) the projection row is first
// formed as the bf16 rounding of the sum of S fp32 partial rows and stored
// into qkv.
hipError_t launch_rope_kv(int dtype, void* qkv, int T, const int* positions, const float2* table,
                          int nq, int nkv, int d, const int* block_table, int max_blocks, int q_len,
                          void* k_cache, void* v_cache, hipStream_t s, const float* part = nullptr,
                          int S = 0);

// attention.hip
struct AttnPlan {
  int parts;        // key partitions per query (1 = no split)
  int part_len;     // keys per partition
  size_t ws_bytes;  // fp32 partial results
};
AttnPlan attention_plan(int T, int nq, int nkv, int d, int q_len, int max_seq_len, int num_cus);
hipError_t launch_attention(int dtype, const void* q, int ldq, int T, const int* positions, int nq,
                            int nkv, int d, const void* k_cache, const void* v_cache,
                            const int* block_table, int max_blocks, int q_len,
                            const AttnPlan& plan, float* partials, void* out, hipStream_t s,
                            hipEvent_t mid_event);

// attention_decode.hip (bf16, one query token per sequence)
hipError_t launch_decode_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                        int d, const void* k_cache, const void* v_cache, const int* block_table,
                                        int max_blocks, int q_len, int part_len, int parts, float* partials,
                                        void* out, hipStream_t s);

// attention_prefill.hip (bf16, q_len > 1, G in {4, 8, 16})
bool prefill_attention_supported(int nq, int nkv, int d);
hipError_t launch_prefill_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                         int d, const void* k_cache, const void* v_cache, const int* block_table,
                                         int max_blocks, int q_len, void* out, hipStream_t s);

}  // namespace llk
