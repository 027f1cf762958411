/*
 * ll.h — C ABI of the little-lm training-step hot path on AMD Instinct MI355X (gfx950).
 *
 * One decoder layer of the little-lm 3.8B model, forward and backward, its FP8 e4m3 tensorwise
 * quantiser, the fused linear cross-entropy LM-head loss, and the whole model (embedding, layers,
 * final norm, head) for one micro-batch built from them. The model is stated on the
 * "hn.213312.xyz translation" page (section 设置 / Setup: RMSNorm, RoPE, GQA 24 query / 8 KV
 * heads, relu^2 MLP, QK-norm, logit softcap, per-layer learnable residual scalars, ResFormer-style
 * value embeddings) and on the "youdonthavefriends cost analysis" page (section "config
 * appendix": hidden 3072, intermediate 12288 non-gated, head_dim 128, rope_theta 10000,
 * rms_norm_eps 1e-6, vocab padded 50257 -> 50304, bf16, FP8 on, loss
 * LigerFusedLinearCrossEntropyLoss(softcap=15.0)).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to caller-owned memory, 16-byte aligned, row-major,
 *     densely packed unless a leading dimension is given. The library never allocates device
 *     memory (ll_fp8_quant_tensorwise_noalloc's scratch is a static device array, below). State
 *     kept between calls: the text of the last error; and, set only through the test entry points
 *     of ll_testing.h, a process-wide GEMM block-configuration override (llt_set_gemm_config,
 *     0 = automatic, the default) and an optional launch trace (llt_trace_begin/end), which the
 *     calls here read.
 *   - `stream` is a hipStream_t (NULL = the default stream). All work is enqueued on it with no
 *     host synchronisation; outputs are valid once the stream has reached the enqueued work.
 *   - Every call validates its arguments before enqueuing anything and returns an ll_status.
 *     A failed validation enqueues nothing. A launch failure returns LL_ERR_HIP; the HIP error
 *     text is then in ll_last_error().
 *   - Values that are not finite in the inputs give non-finite or unspecified results (the e4m3
 *     quantiser turns a NaN into the NaN code 0x7F so that it reaches the FP8 GEMMs). Token ids
 *     outside [0, rows of their table) select nothing: the embedding and value-embedding gathers
 *     add zero rows and their gradient scatters skip them. Targets outside [0, v) other than
 *     ignore_index give unspecified results (they are not checked on the device).
 *   - Calls that share a workspace, `saved` buffer or output on one stream run in order; the
 *     caller must not run two calls that share such memory on different streams at once.
 */
#ifndef LL_H_
#define LL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LL_OK = 0,
  LL_ERR_INVALID_ARG = 1,   /* null pointer, bad shape or leading dimension, misaligned pointer */
  LL_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. fp8 with fp32, head_dim not 64/128) */
  LL_ERR_WORKSPACE = 3,     /* workspace or saved buffer smaller than the size query returns */
  LL_ERR_HIP = 4            /* HIP launch/runtime error; see ll_last_error() */
} ll_status;

typedef enum { LL_F32 = 0, LL_BF16 = 1 } ll_dtype;

/* MLP of the layer: the run's non-gated relu^2 MLP, or the gated SwiGLU MLP it replaced
 * [linlog.top article, 吞吐量优化: removing the SwiGLU gate (three matmuls -> two) raised
 * throughput; manulx summary: SwiGLU's intermediate ratio 2.75 vs 4 for relu^2]. */
typedef enum { LL_MLP_RELU2 = 0, LL_MLP_SWIGLU = 1 } ll_mlp_kind;

/* Static shape and precision of one decoder layer. */
typedef struct {
  int32_t dtype;            /* ll_dtype of activations and weight matrices */
  int32_t fp8_mlp;          /* 1: the three GEMMs of each MLP linear take e4m3 operands (LL_BF16 only) */
  int64_t batch, seq;       /* tokens = batch * seq; positions restart at 0 in every batch row */
  int32_t d_model;          /* D */
  int32_t n_q_heads;        /* Hq */
  int32_t n_kv_heads;       /* Hkv; Hq must be a multiple of Hkv (q head h reads kv head h / (Hq/Hkv)) */
  int32_t head_dim;         /* Dh: 64 or 128 */
  int32_t d_ff;             /* F (4 * D in the model) */
  float rms_eps;            /* 1e-6: block RMSNorms and QK-norm */
  float rope_theta;         /* 10000 */
  int32_t has_value_embed;  /* 1 on value-embedding layers (v += ve_table[token_ids]) */
  int64_t ve_rows;          /* rows of ve_table (padded vocabulary, 50304) */
  int32_t mlp_kind;         /* ll_mlp_kind. LL_MLP_SWIGLU: w_fc is [2 d_ff, D] (gate rows, then up
                               rows), a = silu(x w_gate^T) (x w_up^T), m = a w_proj^T; bf16 / fp32
                               GEMMs only (fp8_mlp must be 0); d_ff = 8448 = 2.75 D in the variant */
} ll_layer_cfg;

/* Parameters of one layer (read only). Matrices are in cfg.dtype; gains and scalars are fp32. */
typedef struct {
  const void* attn_norm_w;   /* fp32 [D]: gain of the pre-attention RMSNorm */
  const void* w_qkv;         /* [(Hq + 2 Hkv) * Dh, D]: q rows, then k rows, then v rows, head-major */
  const void* w_o;           /* [D, Hq * Dh] */
  const void* mlp_norm_w;    /* fp32 [D]: gain of the pre-MLP RMSNorm */
  const void* w_fc;          /* [F, D] ([2F, D] for SwiGLU) */
  const void* w_proj;        /* [D, F] */
  const void* ve_table;      /* [ve_rows, Hkv * Dh] in cfg.dtype, or NULL when !has_value_embed */
  const float* resid_attn;   /* device fp32 scalar a_attn:  h = x + a_attn * attention branch */
  const float* resid_mlp;    /* device fp32 scalar a_mlp:   y = h + a_mlp * MLP branch */
} ll_layer_params;

/* Gradients of one layer. Matrices are written in cfg.dtype; gains, scalars and the
 * value-embedding table in fp32 (the table's gradient is a scatter-add of the rows the token ids
 * pick).
 * accumulate = 0: every gradient is overwritten (the table is zeroed, then scattered into);
 * accumulate = 1: every gradient is added to what the buffers hold (gradient accumulation over the
 * micro-batches of one optimizer step [youdonthavefriends cost analysis, "config appendix": 7
 * accumulation steps of 20 x 2048 tokens per GPU]): each matrix element is rounded once,
 * round(old + new), in cfg.dtype (bf16 master weights carry bf16 gradients [linlog.top article,
 * 吞吐量优化: bf16 主权重]). */
typedef struct {
  void* attn_norm_w;   /* fp32 [D] */
  void* w_qkv;
  void* w_o;
  void* mlp_norm_w;    /* fp32 [D] */
  void* w_fc;
  void* w_proj;
  float* ve_table;     /* fp32 [ve_rows, Hkv * Dh] or NULL */
  float* resid_attn;   /* fp32 scalar */
  float* resid_mlp;    /* fp32 scalar */
  int32_t accumulate;  /* 0: overwrite, 1: add into the existing gradients */
} ll_layer_grads;

/* Bytes of the opaque `saved` buffer that ll_layer_fwd fills and ll_layer_bwd reads, and of the
 * scratch workspace either call needs. Return 0 if cfg is invalid. */
size_t ll_layer_saved_bytes(const ll_layer_cfg* cfg);
size_t ll_layer_workspace_bytes(const ll_layer_cfg* cfg);

/* Forward of one decoder layer [hn.213312.xyz translation, 设置 / Setup; youdonthavefriends cost
 * analysis, "config appendix"]:
 *   xn = RMSNorm(x) g1;  [q|k|v] = xn W_qkv^T;  v += ve_table[token_ids] (value-embedding layers);
 *   q^ = RoPE(QKnorm(q)), k^ = RoPE(QKnorm(k));  o = causal softmax(q^ k^T / sqrt(Dh)) v (GQA);
 *   h = x + a_attn (o W_o^T);  hn = RMSNorm(h) g2;  y = h + a_mlp (relu(hn W_fc^T)^2 W_proj^T),
 * with the MLP GEMMs on dynamically quantised e4m3 operands when cfg.fp8_mlp.
 *   x, y: [batch * seq, D] in cfg.dtype (y must not alias x).  token_ids: int32 [batch * seq]
 *   (required on value-embedding layers, else may be NULL).  saved: >= ll_layer_saved_bytes.
 *   ws: >= ll_layer_workspace_bytes. */
int ll_layer_fwd(const ll_layer_cfg* cfg, const ll_layer_params* p, const void* x,
                 const int32_t* token_ids, void* y, void* saved, size_t saved_bytes, void* ws,
                 size_t ws_bytes, void* stream);

/* Backward of one decoder layer, given dy = dL/dy [batch * seq, D] (cfg.dtype) and the `saved`
 * buffer of the matching ll_layer_fwd call (same cfg, params, x and token_ids). Writes
 * dx = dL/dx [batch * seq, D] (must not alias dy or x) and the gradients in `g`. The FP8 path
 * quantises dL/dm and dL/du and runs the two backward GEMMs of each MLP linear (input gradient,
 * weight gradient) on e4m3 operands, straight-through [hn.213312.xyz translation, 提升吞吐量 /
 * Increasing throughput: three FP8 GEMMs, one forward and two backward]. */
int ll_layer_bwd(const ll_layer_cfg* cfg, const ll_layer_params* p, const void* x,
                 const int32_t* token_ids, const void* saved, size_t saved_bytes, const void* dy,
                 void* dx, const ll_layer_grads* g, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of ll_fused_lce_fwd_bwd for these sizes (0 if invalid). */
size_t ll_fused_lce_workspace_bytes(int32_t dtype, int64_t n, int32_t d, int64_t v, int64_t token_chunk,
                                    int32_t vocab_tile);

/* Fused linear cross-entropy with tanh logit softcap [youdonthavefriends cost analysis,
 * "Increasing throughput" and "config appendix"; hn.213312.xyz translation, 提升吞吐量: the LM
 * head matmul is chunked inside the loss and the (n, v) logits are never materialised]:
 *   z = hidden weight^T, c = softcap tanh(z / softcap), lse_i = log sum_j exp(c_ij),
 *   softcap in (0, 60] (the row sums of exp(c) keep no running maximum: |c| <= softcap bounds them),
 *   loss = mean over rows with targets_i != ignore_index of (lse_i - c_{i, targets_i}),
 *   dz = grad_scale / n_valid (softmax(c) - onehot) (1 - (c / softcap)^2),
 *   d_hidden = dz weight, d_weight = dz^T hidden.
 *   dtype: LL_F32 or LL_BF16 for hidden, weight, d_hidden, d_weight.
 *   hidden [n, d], weight [v, d] (all v rows take part in the softmax, padded rows included),
 *   targets int32 [n] in [0, v) or == ignore_index.  token_chunk: rows per chunk (memory of the
 *   per-chunk logits is token_chunk * v * 2 bytes (bf16) of ws); 0 picks 10240.
 *   vocab_tile: vocabulary columns per partial row sum of exp(c), the N tile of the logits GEMM:
 *   128 or 256 (0 picks 256).  accumulate_dw: 0 overwrites d_weight, 1 adds into it (one rounding
 *   of old + new; gradient accumulation over micro-batches). With several
 *   chunks d_weight is accumulated in an fp32 buffer of ws and rounded once at the end; when one
 *   chunk holds all n rows the whole contraction is rounded straight into d_weight. With
 *   gradients, ws also holds one transposed copy of weight ([d, v rounded up to 64]).
 *   loss: device fp32 scalar (0 if no row is valid).  lse: device fp32 [n] or NULL.
 *   d_hidden [n, d] and d_weight [v, d]: both NULL (forward only) or both non-NULL (overwritten).
 *   Requires d % 64 == 0 (bf16) / d % 32 == 0 (fp32), v % 8 == 0. */
int ll_fused_lce_fwd_bwd(int32_t dtype, const void* hidden, const void* weight,
                         const int32_t* targets, int64_t n, int32_t d, int64_t v, float softcap,
                         int32_t ignore_index, float grad_scale, int64_t token_chunk, int32_t vocab_tile,
                         int32_t accumulate_dw, float* loss, float* lse, void* d_hidden, void* d_weight,
                         void* ws, size_t ws_bytes, void* stream);

/* Parameters of the whole model (read only). */
typedef struct {
  const void* embed;               /* [vocab, D] in cfg.dtype: token embedding table */
  const ll_layer_params* layers;   /* host array [n_layers]; layers[i].ve_table != NULL makes layer i a
                                      value-embedding layer (table [vocab, Hkv * Dh]) */
  const float* final_norm_w;       /* fp32 [D]: gain of the final RMSNorm */
  const void* head;                /* [vocab, D] in cfg.dtype: untied LM head */
} ll_model_params;

/* Gradients of the whole model. */
typedef struct {
  float* embed;                    /* fp32 [vocab, D] (zeroed, then scattered into; added into with
                                      accumulate) */
  const ll_layer_grads* layers;    /* host array [n_layers], as for ll_layer_bwd (ve_table non-NULL exactly
                                      on the value-embedding layers) */
  float* final_norm_w;             /* fp32 [D], written (added into with accumulate) */
  void* head;                      /* [vocab, D] in cfg.dtype, written (added into with accumulate) */
  int32_t accumulate;              /* 0: overwrite, 1: add into every gradient (the layers' own
                                      accumulate fields are ignored) */
} ll_model_grads;

/* Bytes of the `saved` buffer (activations of every layer) and of the workspace of
 * ll_model_fwd_bwd; 0 if the arguments are invalid. cfg.has_value_embed and cfg.ve_rows are
 * ignored (see below). */
size_t ll_model_saved_bytes(const ll_layer_cfg* cfg, int32_t n_layers, int64_t vocab);
size_t ll_model_workspace_bytes(const ll_layer_cfg* cfg, int32_t n_layers, int64_t vocab, int64_t token_chunk);

/* Forward and backward of the whole little-lm model on one micro-batch [hn.213312.xyz
 * translation, 设置 / Setup, parameter table: token embeddings, 28 decoder layers, 14
 * value-embedding tables on every other layer, untied LM head; youdonthavefriends cost analysis,
 * "config appendix": loss LigerFusedLinearCrossEntropyLoss(softcap=15.0)]:
 *   x_0 = embed[token_ids];  x_{i+1} = layer_i(x_i)  (ll_layer_fwd with cfg, and
 *   has_value_embed = (layers[i].ve_table != NULL), ve_rows = vocab);
 *   hn = RMSNorm(x_L) final_norm_w  (eps cfg.rms_eps; a final norm before the head is the
 *   Llama-style reading, its gain fits the parameter table);
 *   loss, dhn, d_head = ll_fused_lce_fwd_bwd(hn, head, targets, softcap, ignore_index,
 *   grad_scale, token_chunk);
 * then the backward chain: final-norm backward, ll_layer_bwd from the last layer to the first,
 * and d_embed[token_ids[n]] += dL/dx_0[n] in fp32. token ids outside [0, vocab) select zero rows
 * (embedding and value embeddings) and receive no gradient; targets follow ll_fused_lce_fwd_bwd. token_ids, targets: int32 [cfg.batch * cfg.seq] device arrays; loss:
 * device fp32 scalar. */
int ll_model_fwd_bwd(const ll_layer_cfg* cfg, int32_t n_layers, int64_t vocab, const ll_model_params* p,
                     const int32_t* token_ids, const int32_t* targets, float softcap, int32_t ignore_index,
                     float grad_scale, int64_t token_chunk, float* loss, const ll_model_grads* g, void* saved,
                     size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- optimizer step
 * The training run's optimizer [youdonthavefriends cost analysis, "config appendix": matrix
 * parameters take Muon (lr 0.02, momentum 0.95, weight decay 0), the embeddings, LM head,
 * value-embedding tables and scalars take AdamW with per-group lr, betas (0.8, 0.995 | 0.96 |
 * 0.95), eps 1e-10 and weight decay; linlog.top article, 吞吐量优化: bf16 master weights, so the
 * parameters and the optimizer state beside them are bf16]. Both calls update in place. */

/* Workspace bytes of ll_muon_step for a [rows, cols] matrix (0 if invalid): rows * cols bf16 for
 * the momentum output, 2 min(rows, cols) max(rows, cols) bf16 for the iterates and
 * 2 min(rows, cols)^2 bf16 for the Gram matrices. */
size_t ll_muon_workspace_bytes(int64_t rows, int64_t cols);

/* One Muon step of a matrix parameter w [rows, cols] (bf16, row-major) with gradient grad and
 * momentum buffer momentum_buf (both bf16 [rows, cols]):
 *   buf = round(momentum buf + grad);  u = round(grad + momentum buf) if nesterov, else buf;
 *   X_0 = round(u / (||u||_F + 1e-7)), transposed when rows > cols (X is [min, max]);
 *   ns_steps times: A = round(X X^T);  B = round(b A + c A A);  X = round(a X + B X),
 *   (a, b, c) = (3.4445, -4.7750, 2.0315): the quintic Newton-Schulz orthogonalisation published
 *   with Muon (K. Jordan, "Muon: An optimizer for hidden layers in neural networks", 2024; the
 *   pages name Muon but not its constants), 5 steps in the published recipe;
 *   w = round(w (1 - lr weight_decay) - lr sqrt(max(1, rows / cols)) X), X back in w's orientation.
 * dtype must be LL_BF16; rows and cols multiples of 64 (<= 65536). The GEMMs run on bf16 MFMA with
 * fp32 accumulation; every stored iterate is rounded to bf16 once. */
int ll_muon_step(int32_t dtype, void* w, const void* grad, void* momentum_buf, int64_t rows, int64_t cols,
                 float lr, float momentum, int32_t nesterov, float weight_decay, int32_t ns_steps, void* ws,
                 size_t ws_bytes, void* stream);

/* One AdamW step of n parameters (decoupled weight decay, bias-corrected moments, as torch.optim.AdamW):
 *   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
 *   p = p (1 - lr weight_decay) - lr (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps),
 * step = 1 for the first update. param, exp_avg and exp_avg_sq are in param_dtype (LL_BF16 for bf16
 * master weights, each rounded once where stored, or LL_F32), grad in grad_dtype. No alignment
 * beyond 16 bytes and any n >= 0. */
int ll_adamw_step(int32_t param_dtype, int32_t grad_dtype, void* param, const void* grad, void* exp_avg,
                  void* exp_avg_sq, int64_t n, float lr, float beta1, float beta2, float eps, float weight_decay,
                  int64_t step, void* stream);

/* Workspace bytes of ll_fp8_quant_tensorwise (a few bytes for the amax). */
size_t ll_fp8_quant_workspace_bytes(void);

/* Dynamic tensorwise e4m3fn quantisation of x [rows, cols] (leading dimension ld >= cols, a
 * multiple of 8; cols a multiple of 16; elements of in_dtype) [linlog.top article, 吞吐量优化:
 * torch._scaled_mm with dynamic tensorwise scaling; the constants are this library's reading]:
 *   amax = max|x|;  scale = 2^floor(log2(fl32(448 / max(amax, 1e-12))));  inv_scale = 1 / scale;
 *   q = e4m3fn_round_nearest_even(clamp(fl32(x * scale), -448, 448)).
 * The power-of-two scale keeps x * scale exact and does not move when amax changes by a rounding
 * error, so two implementations that agree up to rounding pick the same scale.
 * q: uint8 [rows, cols] or NULL; q_t: uint8 [cols, rows] (the transpose) or NULL; scale and
 * inv_scale: device fp32 scalars. Results are bit-exact and independent of launch order. */
int ll_fp8_quant_tensorwise(int32_t in_dtype, const void* x, int64_t rows, int64_t cols,
                            int64_t ld, uint8_t* q, uint8_t* q_t, float* scale, float* inv_scale,
                            void* ws, size_t ws_bytes, void* stream);

/* ll_fp8_quant_tensorwise for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments without the
 * workspace, the same results bit for bit. Its scratch (the amax accumulator and the two scales,
 * 16 bytes) lives in a static 256-byte device array, one per GPU, held until the process ends;
 * the tensor-size limits are those of ll_fp8_quant_tensorwise (the scratch does not grow with the
 * tensor). Every call on one GPU shares that array and leaves its contents behind (each call
 * clears the amax itself before use): calls that overlap on one GPU, on different streams or
 * threads, race and must be ordered by the caller. No hipMalloc, hipFree or other allocation. */
int ll_fp8_quant_tensorwise_noalloc(int32_t in_dtype, const void* x, int64_t rows, int64_t cols,
                                    int64_t ld, uint8_t* q, uint8_t* q_t, float* scale,
                                    float* inv_scale, void* stream);

/* Text of a status code, and a description of the last error raised by this library in the
 * calling thread (empty if none). */
const char* ll_status_string(int status);
const char* ll_last_error(void);

/* Library version (major * 10000 + minor * 100 + patch). */
int ll_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LL_H_ */
