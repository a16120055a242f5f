/*
 * llama_layer.h -- C ABI of an MI355X (gfx950) library that runs the forward
 * pass of one Llama-architecture decoder layer, structured as vLLM's llama.py
 * structures it.
 *
 * The layer, step by step, as the pages describe it:
 *   1. input_layernorm: RMSNorm with the residual add fused in.  With no
 *      incoming residual the hidden state itself becomes the residual;
 *      otherwise hidden + residual becomes the residual and its normalised
 *      value the hidden state.  (page "LLama", hotelren.com/news/2693952,
 *      section "3 input_layernorm (RMSNorm)")
 *   2. merged qkv projection, split into q, k, v in that order; RoPE on q and
 *      k only; attention; o_proj.  (same page, section "4 LlamaAttention";
 *      "vLLM Llama 代码解析", yeyulingfeng.com/a/605382, section
 *      "4.LlamaAttention")
 *   3. the new k, v are written into the layer's paged KV cache before the
 *      attention reads it through the block table.  ("模型库与算子层 — 代码走读",
 *      vllm-learning.pages.dev/topics/model-layers/code-walkthrough, section
 *      "Attention 层")
 *   4. post_attention_layernorm (add + RMSNorm), merged gate_up projection,
 *      SiluAndMul = silu(x[:d]) * x[d:], down_proj.  ("LLama" page, sections
 *      "post_attention_layernorm" and "LlamaMLP")
 *   5. the layer returns the pair (hidden, residual) that the next layer takes.
 *      (yeyulingfeng page, section "2.1 LlamaModel.forward()")
 *
 * Configuration fields carry the names of the model's config.json (the
 * DeepSeek-R1-Distill-Llama-70B config printed on the "LLama" page).
 *
 * Conventions for every call below:
 *   - "device" pointers point into GPU memory of the current HIP device;
 *     "host" pointers into ordinary CPU memory.
 *   - Linear weights are row-major [out_features, in_features] and y = x W^T
 *     (vllm-learning page, section "Linear 层", F.linear).  Packed weights
 *     follow vLLM's packed_modules_mapping (yeyulingfeng page, section 1):
 *     qkv_proj rows are [q heads | k heads | v heads], head h owning rows
 *     h*head_dim .. h*head_dim+head_dim-1; gate_up_proj rows are [gate | up].
 *   - Activations are row-major [num_tokens, features] in the layer dtype.
 *   - Every call returns a llama_status; on failure the thread's last error
 *     message is available from llama_layer_last_error().  Argument errors
 *     are detected on the host before anything is enqueued.
 *   - Work is enqueued on the HIP stream passed as `stream` (NULL = the null
 *     stream); no call synchronises the host with the device unless stated.
 */
#ifndef LLAMA_LAYER_H
#define LLAMA_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLAMA_API __attribute__((visibility("default")))

typedef enum {
  LLAMA_OK = 0,
  LLAMA_ERR_INVALID_ARGUMENT = 1, /* a size, pointer or combination that is wrong */
  LLAMA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. hidden_act != "silu") */
  LLAMA_ERR_OUT_OF_MEMORY = 3,    /* a device allocation inside create() failed */
  LLAMA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} llama_status;

typedef enum { LLAMA_DTYPE_BF16 = 0, LLAMA_DTYPE_FP32 = 1 } llama_dtype;

/* Model configuration (host memory, owned by the caller, read during create
 * only).  Constraints checked by llama_layer_config_validate:
 *   hidden_act must be "silu" (the LlamaMLP constructor on the "LLama" page
 *     raises ValueError for anything else)            -> LLAMA_ERR_UNSUPPORTED
 *   attention_bias, mlp_bias must be 0 (the config has none) -> UNSUPPORTED
 *   rope_type "default" or "llama3"                    -> else UNSUPPORTED
 *   llama3: rope_factor >= 1, high_freq_factor > low_freq_factor > 0,
 *     original_max_position_embeddings > 0             -> else INVALID_ARGUMENT
 *   num_attention_heads % num_key_value_heads == 0     -> else INVALID_ARGUMENT
 *   head_dim in {64, 128}; kv_block_size == 16         -> else UNSUPPORTED
 *   bf16: hidden_size, intermediate_size and (heads + 2*kv_heads)*head_dim
 *     multiples of 128, hidden_size and (heads + 2*kv_heads)*head_dim <= 16384;
 *   fp32: hidden_size multiple of 4, hidden_size <= 8192 -> else UNSUPPORTED
 *   all sizes > 0, rms_norm_eps > 0, rope_theta > 1, dtype known
 *                                                      -> else INVALID_ARGUMENT */
typedef struct {
  int32_t hidden_size;
  int32_t num_attention_heads;
  int32_t num_key_value_heads;
  int32_t head_dim;
  int32_t intermediate_size;
  int32_t max_position_embeddings;  /* positions must be < this */
  float rms_norm_eps;
  double rope_theta;
  const char* hidden_act;           /* "silu" */
  const char* rope_type;            /* "default" or "llama3" (NULL = "default") */
  double rope_factor;               /* llama3 rope_scaling.factor */
  double low_freq_factor;           /* llama3 rope_scaling.low_freq_factor */
  double high_freq_factor;          /* llama3 rope_scaling.high_freq_factor */
  int32_t original_max_position_embeddings; /* llama3 rope_scaling field */
  int32_t attention_bias;           /* must be 0 */
  int32_t mlp_bias;                 /* must be 0 */
  int32_t dtype;                    /* llama_dtype of weights, activations, KV cache */
  int32_t kv_block_size;            /* tokens per KV-cache block; must be 16 */
  /* Mixture of experts (the Qwen3-MoE layer: page "LLama", sections
   * "Qwen3MoeForCausalLM" and "Qwen3MoeSparseMoeBlock"; page "模型库与算子层 —
   * 代码走读", section "Fused MoE").  num_experts = 0: the dense LlamaMLP.
   * num_experts > 0: the MLP becomes a sparse block -- a router [E, H] gives
   * each token a logit per expert; its num_experts_per_tok experts with the
   * largest softmax probabilities (equal ones: lower expert first) each run
   * down(silu(x Wg^T) * (x Wu^T)) with their own weights; the outputs are
   * summed weighted by those probabilities, divided by their sum when
   * norm_topk_prob != 0.  bf16 only; num_experts a multiple of 16 up to 256,
   * 1 <= num_experts_per_tok <= min(num_experts, 64), moe_intermediate_size a
   * multiple of 128, hidden_size a multiple of 256      -> else UNSUPPORTED */
  int32_t num_experts;
  int32_t num_experts_per_tok;
  int32_t moe_intermediate_size;
  int32_t norm_topk_prob;
  /* qk_norm != 0: each q and k head is RMS-normalised over head_dim (weights
   * q_norm / k_norm, eps rms_norm_eps) before RoPE, as Qwen3 attention does. */
  int32_t qk_norm;
} llama_layer_config;

/* Device pointers to the layer's weights in the layer dtype:
 *   input_layernorm, post_attention_layernorm  [hidden_size]
 *   qkv_proj      [(heads + 2*kv_heads) * head_dim, hidden_size]
 *   o_proj        [hidden_size, heads * head_dim]
 *   gate_up_proj  [2 * intermediate_size, hidden_size]      (dense layers)
 *   down_proj     [hidden_size, intermediate_size]          (dense layers)
 *   q_norm, k_norm  [head_dim]                              (qk_norm only)
 *   router        [num_experts, hidden_size]                (MoE layers)
 *   experts_gate_up [num_experts, 2 * moe_intermediate_size, hidden_size],
 *                 each expert [gate | up]: the fused layer's w13 (MoE layers)
 *   experts_down  [num_experts, hidden_size, moe_intermediate_size]: w2
 * Pointers a configuration does not use may be NULL.                        */
typedef struct {
  const void* input_layernorm;
  const void* qkv_proj;
  const void* o_proj;
  const void* post_attention_layernorm;
  const void* gate_up_proj;
  const void* down_proj;
  const void* q_norm;
  const void* k_norm;
  const void* router;
  const void* experts_gate_up;
  const void* experts_down;
} llama_layer_weights;

/* One layer's paged KV cache (device memory owned by the caller), two planes
 * in the layer dtype, each num_blocks blocks of 16 token slots per KV head:
 *   k  [num_blocks][kv_heads][16][head_dim]   (a slot's K row contiguous)
 *   v  [num_blocks][kv_heads][head_dim][16]   (the 16 slots of one V
 *                                              component contiguous)
 * Token position p of sequence b lives in block block_table[b][p / 16],
 * slot p % 16.  K is stored after RoPE.  The V plane keeps the 16 slots of a
 * component together so that attention reads V as the key-major operand of
 * its P.V product with whole-vector loads (the layout vLLM's paged attention
 * uses for V).  It replaces a V plane ordered like K ([blocks][kv_heads][16]
 * [head_dim]), which would make every P.V operand a gather of 2-byte values
 * from 16 different slot rows.                                              */
typedef struct {
  void* k;
  void* v;
  int32_t num_blocks;
} llama_kv_cache;

typedef struct llama_layer llama_layer;

/* Host-only check of a configuration; touches no GPU. */
LLAMA_API llama_status llama_layer_config_validate(const llama_layer_config* config);

/* Builds a layer: validates `config`, copies the weights into memory the
 * library owns (gate_up_proj is re-ordered so that each 32-row group holds 16
 * gate rows followed by the matching 16 up rows), and builds the RoPE
 * cos/sin table [max_position_embeddings][head_dim/2] (angles and their
 * cosines/sines in double precision on the host, stored as float).  Runs on
 * `stream`; the caller may free its weight buffers once `stream` has passed
 * this call.  *out receives the handle, which is immutable afterwards and may
 * be shared by concurrent forwards on different streams.
 * Errors: INVALID_ARGUMENT / UNSUPPORTED as for validate, or NULL pointers;
 * OUT_OF_MEMORY; HIP. */
LLAMA_API llama_status llama_layer_create(const llama_layer_config* config, const llama_layer_weights* weights,
                                void* stream, llama_layer** out);

/* Bytes of device workspace llama_layer_forward needs for a call with these
 * host-side bounds (0 on a NULL layer or non-positive sizes). */
LLAMA_API size_t llama_layer_workspace_bytes(const llama_layer* layer, int32_t num_tokens, int32_t num_seqs,
                                   int32_t max_seq_len);

/* One forward of the layer.
 *   hidden       [T, H] device, the layer input.
 *   residual     [T, H] device, or NULL for the first layer (residual := hidden).
 *   positions    [T] int32 device, position of each token in its sequence.
 *   num_tokens   T > 0.
 *   kv_cache     this layer's cache; the K/V of the T new tokens are written
 *                at their positions, then attention reads positions 0..p.
 *   block_table  [num_seqs][max_blocks_per_seq] int32 device.
 *   seq_lens     [num_seqs] int32 device: each sequence's KV length after
 *                this call (its cached context plus its new tokens).
 *   query_start_loc  NULL: the T tokens are num_seqs equal runs of
 *                T / num_seqs consecutive rows, one run per sequence.
 *                Otherwise [num_seqs + 1] int32 device: sequence b owns rows
 *                query_start_loc[b] .. query_start_loc[b+1] - 1, with
 *                query_start_loc[0] = 0, query_start_loc[num_seqs] = T and at
 *                least one row per sequence.  This is a mixed batch: chunked
 *                prefill on a cached context next to decode sequences (one
 *                row each) in one call, the per-call metadata that the
 *                attention backend of the vllm-learning page
 *                "模型库与算子层 — 代码走读" (section "Attention 层") passes
 *                with the block table.  At most 4096 sequences.  A mixed
 *                batch adds one small kernel that maps rows to sequences.
 *                Either way the run of sequence b holds positions
 *                seq_lens[b] - n_b .. seq_lens[b] - 1 in order (n_b its rows).
 *   max_seq_len  host-side upper bound of seq_lens (sizes the launch).
 *   hidden_out, residual_out  [T, H] device: the output pair.  residual_out
 *                = (hidden + residual) + o_proj(attention) (the stream value
 *                after attention), hidden_out = down_proj(SiluAndMul(
 *                gate_up_proj(RMSNorm(residual_out)))), or the sparse MoE
 *                block of RMSNorm(residual_out) in an MoE layer; each
 *                expert's weighted output is rounded to the layer dtype
 *                before the sum over a token's experts.  hidden_out may alias
 *                hidden and residual_out may alias residual; the two outputs
 *                must not alias each other.
 *   workspace    >= llama_layer_workspace_bytes(layer, T, num_seqs, max_seq_len)
 *                bytes of device memory, 256-byte aligned.
 * The call writes only hidden_out, residual_out, the new tokens' KV slots and
 * the workspace.  Preconditions on device data (block ids < num_blocks,
 * positions < max_position_embeddings and consistent with seq_lens, the
 * query_start_loc conditions above) are not checked on the device by
 * default; a query_start_loc that breaks them gives wrong rows, but the row
 * map stays inside [0, T) and [0, num_seqs).  With the environment variable
 * LLAMA_DEBUG=1 (read at each call) the call first checks them with one
 * kernel and synchronises the stream: a broken condition returns
 * INVALID_ARGUMENT naming it, before anything is written.  The check is
 * skipped while the stream is being captured into a graph.
 * Errors: INVALID_ARGUMENT (NULL pointer; T % num_seqs != 0 with
 * query_start_loc NULL; T < num_seqs; T/num_seqs > max_seq_len; max_seq_len >
 * max_position_embeddings or > 16 * max_blocks_per_seq; aliasing outputs),
 * UNSUPPORTED (more than 4096 sequences in a mixed batch), HIP. */
LLAMA_API llama_status llama_layer_forward(llama_layer* layer, const void* hidden, const void* residual,
                                 const int32_t* positions, int32_t num_tokens,
                                 const llama_kv_cache* kv_cache, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 const int32_t* query_start_loc, int32_t num_seqs,
                                 int32_t max_seq_len, void* hidden_out, void* residual_out,
                                 void* workspace, void* stream);

/* llama_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Arguments, results and errors as llama_layer_forward, without
 * the workspace: the forward's intermediate tensors live in a device array
 * of 64 MiB that the library holds on each GPU it runs on, from module load
 * until the process ends (enough for decode batches of up to 64 sequences at
 * 32768-token contexts on the 70B layer).  The call makes no allocation of
 * any kind.  Every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (other streams, other threads) race; the caller
 * serialises them.  Extra errors: INVALID_ARGUMENT when the call would need
 * more than 64 MiB (llama_layer_workspace_bytes tells; use
 * llama_layer_forward with a workspace then), when per-kernel timing is on,
 * or when the current device is not the layer's; HIP when the array's
 * address could not be looked up at create. */
LLAMA_API llama_status llama_layer_forward_noalloc(llama_layer* layer, const void* hidden, const void* residual,
                                                   const int32_t* positions, int32_t num_tokens,
                                                   const llama_kv_cache* kv_cache, const int32_t* block_table,
                                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                                   const int32_t* query_start_loc, int32_t num_seqs,
                                                   int32_t max_seq_len, void* hidden_out, void* residual_out,
                                                   void* stream);

/* Frees the layer's device memory (synchronises the layer's device first;
 * any device may be current, and the caller's current device is kept). */
LLAMA_API void llama_layer_destroy(llama_layer* layer);

/* Message of the calling thread's last failed call ("" if none). */
LLAMA_API const char* llama_layer_last_error(void);

/* ---- the decoder stack ---------------------------------------------------- */

/* num_layers decoder layers followed by the model body's final RMSNorm: page
 * "LLama" (hotelren.com/news/2693952), section "最终 RMSNorm", and page
 * yeyulingfeng.com/a/605382.html, section "2.1 LlamaModel.forward()".  The
 * layers hand (hidden, residual) on, the first with no residual, and the final
 * norm takes hidden + residual: out = RMSNorm(hidden_N + residual_N; w_final).
 * There is no embedding and no lm_head: the input is the embedded hidden state. */
typedef struct llama_stack llama_stack;

/* weights: host array of num_layers layer weight sets (as for
 * llama_layer_create); final_norm: [H] device.  The stack copies everything;
 * the caller may free its buffers once the call returns.  Errors as
 * llama_layer_create, plus INVALID_ARGUMENT for num_layers <= 0. */
LLAMA_API llama_status llama_stack_create(const llama_layer_config* config, int32_t num_layers,
                                          const llama_layer_weights* weights, const void* final_norm, void* stream,
                                          llama_stack** out);

/* Workspace bytes of a stack forward with these bounds (0 on bad input). */
LLAMA_API size_t llama_stack_workspace_bytes(const llama_stack* stack, int32_t num_tokens, int32_t num_seqs,
                                             int32_t max_seq_len);

/* One forward through every layer and the final norm.  Arguments as
 * llama_layer_forward, except: kv_caches is a host array of num_layers caches
 * (layer l reads and writes kv_caches[l]); there is no residual input; out
 * [T, H] device receives the final norm's output.  The layers' (hidden,
 * residual) pair lives in the workspace. */
LLAMA_API llama_status llama_stack_forward(llama_stack* stack, const void* hidden, const int32_t* positions,
                                           int32_t num_tokens, const llama_kv_cache* kv_caches,
                                           const int32_t* block_table, int32_t max_blocks_per_seq,
                                           const int32_t* seq_lens, const int32_t* query_start_loc,
                                           int32_t num_seqs, int32_t max_seq_len, void* out, void* workspace,
                                           void* stream);

/* Frees the stack's device memory (synchronises the stack's device first;
 * any device may be current, and the caller's current device is kept). */
LLAMA_API void llama_stack_destroy(llama_stack* stack);

/* A HIP graph of one llama_stack_forward with exactly these arguments,
 * captured on `stream` (which must not be the default stream) and
 * instantiated.  The graph keeps the pointers, not the contents: between
 * launches the caller may rewrite hidden, positions, seq_lens, block_table and
 * query_start_loc in place (same sizes), and each launch runs the whole forward
 * on what they then hold.  Per-kernel timing must be off.  Errors:
 * INVALID_ARGUMENT, the forward's own errors (the capture is then abandoned),
 * HIP. */
typedef struct llama_graph llama_graph;
LLAMA_API llama_status llama_stack_graph_create(llama_stack* stack, const void* hidden, const int32_t* positions,
                                                int32_t num_tokens, const llama_kv_cache* kv_caches,
                                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                                const int32_t* seq_lens, const int32_t* query_start_loc,
                                                int32_t num_seqs, int32_t max_seq_len, void* out, void* workspace,
                                                void* stream, llama_graph** graph);
/* Launches the graph on `stream` (asynchronous). */
LLAMA_API llama_status llama_graph_launch(llama_graph* graph, void* stream);
/* Frees the graph (synchronises the graph's device first; any device may
 * be current, and the caller's current device is kept). */
LLAMA_API void llama_graph_destroy(llama_graph* graph);

/* ---- inspection -------------------------------------------------------- */

/* Byte offset and size, inside the workspace of a forward with these bounds,
 * of an intermediate tensor the forward leaves there:
 *   "h"    [T, H]          input_layernorm output
 *   "qkv"  [T, QKV]        qkv projection; after the forward its q part holds
 *                          q after RoPE, its k part k before RoPE
 *   "attn" [T, heads*d]    attention output
 *   "h2"   [T, H]          post_attention_layernorm output
 *   "act"  [T, I]          SiluAndMul output (dense layers)
 *   "router_logits" [T, E] float32, "topk_ids" [T, k] int32 (best first),
 *   "topk_weights" [T, k] float32   the MoE routing (MoE layers)
 *   "moe_sorted" [T*k] int32  the (token, expert) pair p = t*k + slot held by
 *                          each row of moe_act (pairs grouped by expert)
 *   "moe_act"  [T*k, moe_intermediate_size]  each pair's SiluAndMul output,
 *                          in moe_sorted's row order
 *   "moe_part" [T*k, H]    each pair's expert output times its routing
 *                          weight, rounded to the layer dtype, row p = pair p;
 *                          hidden_out[t] is the sum over t's k slots
 * Returns INVALID_ARGUMENT for an unknown name or one the layer lacks. */
LLAMA_API llama_status llama_layer_workspace_tensor(const llama_layer* layer, int32_t num_tokens,
                                          int32_t num_seqs, int32_t max_seq_len, const char* name,
                                          size_t* offset, size_t* bytes);

/* The layer's RoPE table, read-only device memory the layer owns (valid
 * until destroy): table[p * pairs + i] = {cos, sin} (two floats) of the
 * angle p * w_i, angle and cosine/sine computed in double precision and
 * rounded once to float, for p < *num_positions (max_position_embeddings) and
 * pair i < *pairs (head_dim / 2).  The RoPE kernel rotates the pair
 * (x0, x1) = (x_i, x_{i + head_dim/2}) of a head at position p with it as
 *   y0 = fmaf(x0, cos, -(x1 * sin)),  y1 = fmaf(x1, cos, x0 * sin)
 * in float, each rounded once to the layer dtype; the K written to the cache
 * is exactly that.  Errors: INVALID_ARGUMENT for NULL arguments. */
LLAMA_API llama_status llama_layer_rope_table(const llama_layer* layer, const void** table, int32_t* num_positions,
                                              int32_t* pairs);

/* Per-kernel timing.  While enabled, every launch of a forward is bracketed
 * by HIP events on the forward's stream.  llama_layer_timing_read waits for
 * the recorded events, writes up to `cap` entries (kernel name, total
 * milliseconds, launch count) accumulated since the last read, clears them and
 * returns the number of distinct kernels (or -1 on error). */
LLAMA_API llama_status llama_layer_set_timing(llama_layer* layer, int32_t enable);
LLAMA_API int32_t llama_layer_timing_read(llama_layer* layer, const char** names, double* total_ms,
                                int64_t* counts, int32_t cap);

/* ---- single steps (the kernels the forward launches), for testing ------ */

typedef enum {
  LLAMA_EPI_STORE = 0,    /* out[M, N]  = x W^T                              */
  LLAMA_EPI_ADD = 1,      /* out[M, N] += x W^T   (out holds the addend)      */
  LLAMA_EPI_SILU_MUL = 2  /* W is a re-ordered gate_up weight [2N, K] (see
                             llama_op_reorder_gate_up); out[M, N] =
                             silu(x W_gate^T) * (x W_up^T)                    */
} llama_epilogue;

/* y = x W^T with an epilogue.  x [M, K], W [N or 2N, K], out [M, N], all
 * device, row-major, dtype `dtype`, 16-byte aligned; fp32 accumulation.
 * bf16 needs K % 64 == 0 and W's row count (N, or 2N for SILU_MUL) % 128 == 0;
 * fp32 takes any sizes and, for SILU_MUL, W in the plain [gate | up] order.
 * M <= 128 runs the weight-streaming kernel the decode path uses, larger M the
 * tiled kernel of the prefill path.  Errors: INVALID_ARGUMENT (NULL, sizes,
 * alignment), HIP. */
LLAMA_API llama_status llama_op_linear(int32_t dtype, const void* x, const void* w, int32_t M, int32_t N,
                             int32_t K, int32_t epilogue, void* out, void* stream);

/* Re-orders a bf16 [gate | up] weight [2I, K] (device) into the layout the
 * bf16 SILU_MUL epilogue reads: 32-row group g holds gate rows 16g..16g+15
 * then up rows 16g..16g+15.  I % 16 == 0.  dst must not alias src. */
LLAMA_API llama_status llama_op_reorder_gate_up(const void* src, int32_t intermediate, int32_t K, void* dst,
                                      void* stream);

/* RMSNorm with optional fused add over `rows` rows of width `hidden`:
 *   residual != NULL: r = x + residual, residual_out = r (dtype-rounded),
 *                     normed = r / sqrt(mean(r^2) + eps) * w
 *   residual == NULL and residual_out != NULL: residual_out = x (bit copy),
 *                     normed = norm(x)
 *   both NULL: normed = norm(x).   All pointers device. */
LLAMA_API llama_status llama_op_add_rmsnorm(int32_t dtype, const void* x, const void* residual, const void* w,
                                  float eps, int32_t rows, int32_t hidden, void* normed,
                                  void* residual_out, void* stream);

/* ---- measurement ------------------------------------------------------ */

/* Reads `bytes` of device memory at src (a multiple of 16, 16-byte aligned)
 * and nothing else: each of `workgroups` workgroups of `threads` threads (a
 * multiple of 64, at most 1024) streams one contiguous region with 16-byte
 * loads, several in flight per lane, and writes one 32-bit word per thread to
 * sink [workgroups * threads] (device) so the loads are kept.  nontemporal
 * != 0 gives the loads the nontemporal hint, as the decode path's weight and
 * KV streams carry it.  Its rate is the HBM read ceiling the streaming
 * kernels of the decode path are measured against.  Errors:
 * INVALID_ARGUMENT, HIP. */
LLAMA_API llama_status llama_diag_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t threads,
                                              int32_t nontemporal, void* sink, void* stream);

/* The same reads gathered by block, as the decode attention reads a paged
 * cache: src holds src_bytes / block_bytes blocks of block_bytes bytes (a
 * multiple of 1024, at most 16384); block_ids [num_ids] (int32, device) lists
 * the blocks to read, each in [0, src_bytes / block_bytes) -- the caller's
 * guarantee, not checked on the device.  Each of `workgroups` workgroups of
 * block_bytes / 16 threads reads a contiguous range of the list, one 16-byte
 * word per thread and block, several blocks in flight, and writes one 32-bit
 * word per thread to sink [workgroups * block_bytes / 16] (device).
 * nontemporal as llama_diag_stream_read.  Errors: INVALID_ARGUMENT, HIP. */
LLAMA_API llama_status llama_diag_block_read(const void* src, size_t src_bytes, const int32_t* block_ids,
                                             int32_t num_ids, int32_t block_bytes, int32_t workgroups,
                                             int32_t nontemporal, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_LAYER_H */
