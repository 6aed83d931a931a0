/*
 * ga.h -- C ABI of the gated grouped-query causal attention library (gfx950).
 *
 * The library computes the forward pass of one full-attention layer of a
 * Qwen3.5 / Qwen3-Next style model, from already-projected q, k, v and gate
 * logits to the gated concat of the head outputs (the input of W_O):
 *
 *   q_hat = RoPE(RMSNorm(q[b,i,h], w_q), pos[b,i])
 *   k_hat = RoPE(RMSNorm(k[b,j,g], w_k), pos[b,j])        g = floor(h / (H/G))
 *   y     = softmax_j<=i(q_hat . k_hat_j * scale) V          scale = 1/sqrt(d)
 *   out[b,i,h*d + e] = y_e * sigmoid(z)                     (elementwise z[b,i,h,e],
 *                                                            headwise z[b,i,h], or none)
 *
 * Sources (page title, section): "Transformer by Hand · 6. Gated attention",
 * "The formula" (causal softmax(QK^T/sqrt(d)) V), "Four things Qwen3.5 adds to
 * the textbook" (GQA, QK-Norm before RoPE, RoPE on the first quarter of the
 * head, output gate) and "The code: qwen/attention.py" (order of operations
 * and shapes); "Gated Attention：算完注意力，再决定用多少", "门放在哪里？"
 * (gate after SDPA and before W_O; headwise vs elementwise); "多头注意力与 GQA",
 * "分组查询注意力（GQA）" (head h reads KV head floor(h/group)) and
 * "标准多头注意力（MHA）" (decode reads every cached K and V; Q is not cached).
 *
 * Readings of points the pages leave open: RMSNorm is x/sqrt(mean(x^2)+eps)*w
 * with w the effective weight; RoPE rotates pairs (t, t + rot/2) inside the
 * first rot dims by pos * base^(-2t/rot); the causal mask is by token index
 * inside a call; a decode token attends to the cache and to itself.
 *
 * Conventions for every entry point:
 *  - Pointers named as tensors are DEVICE pointers; ``desc`` is a host pointer
 *    read during the call only. ``stream`` is a hipStream_t (NULL = the null
 *    stream). All launches are asynchronous on ``stream``.
 *  - The caller owns every buffer. The library writes only ``out``, the
 *    cache slots named below and the workspace. It keeps no state between
 *    calls; calls on different streams with disjoint outputs may overlap.
 *  - Layouts are row-major, innermost index last:
 *      q [B,n,H,d]  k,v [B,n,G,d]  gate [B,n,H,d] | [B,n,H]  out [B,n,H*d]
 *      caches [B,cap,G,d]  norm weights [d] float32  positions [B,n] int32
 *    All are dense except q and the gate, whose head rows may be spaced
 *    wider (``q_head_stride``, ``gate_head_stride`` in the descriptor), so
 *    that the output of a fused q projection is read in place (see there).
 *    Element type of q, k, v, gate, out and caches is ``desc->dtype``.
 *    bf16 tensors must be 16-byte aligned (a headwise gate: 2-byte), norm
 *    weights 16-byte aligned.
 *  - Errors: shapes, pointers, alignment, capacities and workspace size are
 *    checked on the host before anything is launched; a failed check returns
 *    its status and launches nothing. ``ga_last_error()`` gives a message for
 *    the last failure on the calling thread. Data values are not checked:
 *    NaN and Inf propagate through the arithmetic.
 *  - Empty inputs (batch == 0, or seq_len == 0 for prefill) are a no-op
 *    returning GA_OK.
 */
#ifndef GA_H
#define GA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GA_OK = 0,
  GA_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
  GA_ERR_BAD_SHAPE = 2,    /* a size is negative or inconsistent (e.g. H % G != 0) */
  GA_ERR_BAD_DTYPE = 3,    /* dtype or gate mode out of range */
  GA_ERR_UNSUPPORTED = 4,  /* valid but not implemented (e.g. head_dim > 256) */
  GA_ERR_MISALIGNED = 5,   /* a bf16 tensor is not 16-byte aligned */
  GA_ERR_WORKSPACE = 6,    /* workspace missing or smaller than required */
  GA_ERR_HIP = 7           /* the HIP runtime reported an error at launch */
} ga_status;

typedef enum { GA_BF16 = 0, GA_F32 = 1 } ga_dtype;
typedef enum { GA_GATE_NONE = 0, GA_GATE_HEADWISE = 1, GA_GATE_ELEMENTWISE = 2 } ga_gate_mode;

/* Gate variants ("Gated Attention for Large Language Models ... 论文阅读"):
 * the function of the logits z -- sigmoid (the method's gate), NS-sigmoid
 * 0.5 + 0.5 sigmoid(z) ("第二条机制线索：当前 query 决定的稀疏过滤"), SiLU
 * z sigmoid(z) ("五个门控位置与训练结果总览"), identity z (the additive gate
 * without its SiLU, "第一条机制线索：value 与输出投影之间的非线性") -- ... */
typedef enum { GA_ACT_SIGMOID = 0, GA_ACT_NS_SIGMOID = 1, GA_ACT_SILU = 2, GA_ACT_IDENTITY = 3 } ga_gate_act;
/* ... how it meets the attention output y: y * act(z) or y + act(z) (the
 * additive version, "五个门控位置与训练结果总览") ... */
typedef enum { GA_COMBINE_MUL = 0, GA_COMBINE_ADD = 1 } ga_gate_combine;
/* ... and which dims the logits have: one gate per token shared by every
 * head (Table 1's head-shared gate, "实验规模与参数预算怎样控制") and/or one
 * gate for every token (the input-independent gate, "第一条机制线索"). */
typedef enum { GA_SHARE_HEADS = 1, GA_SHARE_TOKENS = 2 } ga_gate_share;

/* Kernel choice of the prefill attention (ga_prefill, ga_prefill_attention)
 * and of the chunk attention (ga_prefill_chunk*): automatic, or forced, for
 * tests and tuning. A forced kernel that does not serve the shape makes the
 * call fail with GA_ERR_UNSUPPORTED (the chunk path serves only MIRROR and
 * GENERIC). Results of every kernel agree within the parity tolerance. */
typedef enum {
  GA_KERNEL_AUTO = 0,
  GA_KERNEL_WIDE = 1,     /* 256 query rows per workgroup, heaviest blocks first (d = 128) */
  GA_KERNEL_MIRROR = 2,   /* 128 rows from a block and its mirror, two key phases (d = 128, 256) */
  GA_KERNEL_SIMPLE = 3,   /* 128 rows of one block (d = 64, 128, 256) */
  GA_KERNEL_GENERIC = 4   /* one wave per query row (any d <= 256, fp32 or bf16) */
} ga_kernel;
/* Kernels of the backward's dq and dK/dV products: automatic (LDS-staged
 * operands where they serve the shape) or the register-operand kernels for
 * every shape. */
typedef enum { GA_BWD_AUTO = 0, GA_BWD_PLAIN = 1 } ga_bwd_kernel;

typedef struct {
  int32_t batch;        /* B >= 0 */
  int32_t n_q_heads;    /* H >= 1, a multiple of n_kv_heads */
  int32_t n_kv_heads;   /* G >= 1 */
  int32_t head_dim;     /* d, 1..256 */
  int32_t rot_dim;      /* RoPE dims, even, 0..d; 0 = no RoPE (configs: d/4) */
  float rope_base;      /* > 0 when rot_dim > 0 (configs: 10000) */
  float rms_eps;        /* >= 0 (configs: 1e-6) */
  float softmax_scale;  /* 0 = 1/sqrt(head_dim); else used as given (> 0) */
  int32_t dtype;        /* ga_dtype: element type of q/k/v/gate/out/caches */
  int32_t gate_mode;    /* ga_gate_mode */
  /* Head strides (elements) of q and the gate; 0 = dense (d for q and an
   * elementwise gate, 1 for a headwise gate). Element e of head h of token i
   * of sequence b is at ((b*n + i)*H + h) * stride + e: the rows of one
   * token follow each other, so the token stride is H * stride. Nonzero
   * values must be >= d (q, elementwise gate) or >= 1 (headwise gate).
   *
   * Fused q projection ("Transformer by Hand · 6. Gated attention", "Why the
   * gate is packed into q_proj" and "The code: qwen/attention.py": each
   * head's 2d outputs are its query followed by its gate): pass q = qg,
   * gate = qg + d and both strides = 2d. A headwise gate packed as [q | z]
   * per head has stride d + 1.
   *
   * The fused bf16 kernels read q rows and elementwise gate rows in 16-byte
   * pieces: with a q stride or an elementwise gate stride that is not a
   * multiple of 8 the call runs on the generic kernel (same results, no
   * throughput claim), and ga_decode_partials / ga_decode_merge refuse it. */
  int32_t q_head_stride;
  int32_t gate_head_stride;
  /* Gate variants (all 0 = the method's gate: y * sigmoid(z), one gate row
   * per token and head). gate_share changes the gate's dims: with
   * GA_SHARE_HEADS a prefill gate is [B,n,d] | [B,n] (decode [B,d] | [B]),
   * with GA_SHARE_TOKENS it is [H,d] | [H], with both [d] | [1]; its rows
   * are gate_head_stride apart (0 = dense). */
  int32_t gate_act;      /* ga_gate_act */
  int32_t gate_combine;  /* ga_gate_combine */
  int32_t gate_share;    /* ga_gate_share bits */
  /* Per-head RMSNorm of the attention output before the gate (the per-head
   * SDPA-output RMSNorm of "第一条机制线索"): y_h / sqrt(mean(y_h^2) + eps) * w.
   * out_norm_w: DEVICE pointer to [d] float32, 16-byte aligned, or NULL for
   * no norm; it must stay valid until the calls that use it have run. */
  float out_norm_eps;    /* >= 0 */
  const float* out_norm_w;
  int32_t kernel;        /* ga_kernel (0 = automatic) */
  int32_t bwd_kernel;    /* ga_bwd_kernel (0 = automatic) */
} ga_attn_desc;

/* ---- prefill ------------------------------------------------------------ */

/* Name of the kernel ga_prefill_attention runs for this shape (caches of
 * seq_len rows): "wide", "mirror", "simple" or "generic"; "unsupported" when
 * the descriptor forces a kernel that does not serve the shape, "invalid"
 * for a bad descriptor. A static string; the caller does not free it. */
const char* ga_prefill_attention_kernel(const ga_attn_desc* desc, int32_t seq_len);

/* Workspace ga_prefill needs when it is given no KV cache: room for K-hat
 * (B*n*G*d elements, rounded up to 256 bytes). With a KV cache it needs
 * none. Depends on its arguments only. */
size_t ga_prefill_workspace_bytes(const ga_attn_desc* desc, int32_t seq_len);

/* Whole prefill: ga_prefill_keys, then ga_prefill_attention.
 *  q, k, v       [B,n,H,d] / [B,n,G,d] / [B,n,G,d], raw projections.
 *  gate          [B,n,H,d] (elementwise) | [B,n,H] (headwise) | NULL (none).
 *  q_norm_w, k_norm_w  [d] float32 effective RMSNorm weights; NULL = no norm.
 *  positions     [B,n] int32 RoPE positions; NULL = token index 0..n-1.
 *  k_cache, v_cache  optional [B,cache_cap,G,d]: when k_cache is given, K-hat
 *                (normed, rotated, rounded to dtype) is written to slots
 *                [0,n) of k_cache and v to the same slots of v_cache (both
 *                required, cache_cap >= n); the attention then reads K-hat
 *                from the cache and ``workspace`` may be NULL. Without a
 *                cache, K-hat goes to ``workspace`` (16-byte aligned,
 *                ga_prefill_workspace_bytes bytes).
 *  out           [B,n,H*d]. */
ga_status ga_prefill(const ga_attn_desc* desc, int32_t seq_len,
                     const void* q, const void* k, const void* v, const void* gate,
                     const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                     void* k_cache, void* v_cache, int32_t cache_cap,
                     void* workspace, size_t workspace_bytes,
                     void* out, void* stream);

/* First stage of ga_prefill (one kernel): k_hat[b,i,g,:] = RoPE(RMSNorm(k))
 * for i < seq_len into k_hat [B,kv_cap,G,d]; when v_out is not NULL, also
 * copies v into v_out [B,kv_cap,G,d]. kv_cap >= seq_len. */
ga_status ga_prefill_keys(const ga_attn_desc* desc, int32_t seq_len,
                          const void* k, const void* v, const float* k_norm_w,
                          const int32_t* positions, void* k_hat, void* v_out, int32_t kv_cap,
                          void* stream);

/* Second stage of ga_prefill: causal attention of the normed, rotated q
 * against prepared keys, with the gate fused into the epilogue. Automatic
 * kernel choice (bf16): the wide kernel (256 query rows per workgroup; d =
 * 128, rot % 32 == 0, at least 512 token blocks), else the mirrored-block
 * kernel (d in {128, 256}, rot <= d/4, B*n*H < 2^31), else the simple kernel
 * (d in {64, 128, 256}), else the generic kernel; desc->kernel may force one.
 * Needs no workspace.
 *  k_hat  [B,k_cap,G,d] as written by ga_prefill_keys (k_cap >= seq_len).
 *  v      [B,v_cap,G,d] (v_cap >= seq_len; the raw v input has v_cap = n).
 *  k_norm_w  [d] float32: the weights ga_prefill_keys normed k_hat with, or
 *         NULL when k_hat has no such norm. With q_norm_w it bounds every
 *         score (|q_hat . k_hat| <= |q_hat| sqrt(d) max|w_k|), and the fused
 *         kernels then subtract that bound instead of a running row max
 *         (softmax is unchanged by any shift). A k_hat whose rows are longer
 *         than the weights allow still gives correct results as long as its
 *         scores stay within about 2^60 of the bound (exp2 range of fp32). */
ga_status ga_prefill_attention(const ga_attn_desc* desc, int32_t seq_len,
                               const void* q, const void* k_hat, int32_t k_cap,
                               const void* v, int32_t v_cap, const void* gate,
                               const float* q_norm_w, const float* k_norm_w,
                               const int32_t* positions, void* out, void* stream);

/* ---- chunked prefill against a KV cache ---------------------------------- */

/* A chunk of new tokens per sequence, appended after the tokens already in a
 * KV cache: the step between a whole-sequence prefill and decode. The
 * attention mask M is the causal mask in cache slots plus a padding mask
 * ("Gated Attention：算完注意力，再决定用多少", section "门放在哪里？": M is the
 * causal / padding mask); the cached keys and values are read as stored
 * ("多头注意力与 GQA", section "标准多头注意力（MHA）": history K and V are
 * kept and re-read, Q is not). "Transformer by Hand · 6. Gated attention"
 * leaves the state and mask arguments of its forward to a later chapter.
 *
 * For sequence b with L_b = cache_lens[b] tokens cached (K-hat and V in slots
 * [0, L_b) of k_cache / v_cache) and n_b = chunk_lens[b] real rows of the
 * seq_len-row chunk (chunk_lens NULL: n_b = seq_len):
 *  - chunk row i < n_b is token L_b + i: its K-hat = RoPE(RMSNorm(k)) and v go
 *    to slot L_b + i, and its query attends to slots [0, L_b + i];
 *  - rows i >= n_b are padding: no cache slot and no output row is written;
 *  - positions [B,seq_len] are the RoPE positions of the chunk rows (NULL:
 *    L_b + i);
 *  - a sequence with L_b outside [0, max_cache_len] is skipped entirely.
 *  q, k, v       [B,seq_len,H,d] / [B,seq_len,G,d] / [B,seq_len,G,d], raw projections.
 *  gate          as for ga_prefill.
 *  k_cache, v_cache  [B,cache_cap,G,d], cache_cap >= max_cache_len + seq_len,
 *                max_cache_len + seq_len < 2^30.
 *  cache_lens, chunk_lens  device int32 [B] (chunk_lens may be NULL).
 *  out           [B,seq_len,H*d]; rows of padding and skipped sequences are left as they were.
 *  workspace     ga_prefill_chunk_workspace_bytes bytes, 256-byte aligned
 *                (NULL when that is 0).
 * The library does not advance cache_lens (the caller adds n_b afterwards).
 * Errors as for ga_prefill. */
ga_status ga_prefill_chunk(const ga_attn_desc* desc, int32_t seq_len,
                           const void* q, const void* k, const void* v, const void* gate,
                           const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                           void* k_cache, void* v_cache, int32_t cache_cap,
                           const int32_t* cache_lens, const int32_t* chunk_lens, int32_t max_cache_len,
                           void* workspace, size_t workspace_bytes, void* out, void* stream);

/* Workspace of ga_prefill_chunk / ga_prefill_chunk_attention, in bytes
 * (256-byte aligned; NULL is accepted when this is 0). Depends on its
 * arguments only. */
size_t ga_prefill_chunk_workspace_bytes(const ga_attn_desc* desc, int32_t seq_len, int32_t cache_cap,
                                        int32_t max_cache_len);

/* First stage of ga_prefill_chunk (one kernel): writes K-hat and v of the
 * real chunk rows to cache slots [L_b, L_b + n_b). */
ga_status ga_prefill_chunk_keys(const ga_attn_desc* desc, int32_t seq_len,
                                const void* k, const void* v, const float* k_norm_w,
                                const int32_t* positions, const int32_t* cache_lens,
                                const int32_t* chunk_lens, int32_t max_cache_len,
                                void* k_cache, void* v_cache, int32_t cache_cap, void* stream);

/* Second stage of ga_prefill_chunk (one kernel): the chunk's queries against
 * cache slots [0, L_b + i], gated, into out. Expects the chunk's own K-hat
 * and v already in the cache (ga_prefill_chunk_keys). k_norm_w is the weight
 * the cached K-hat was normed with (or NULL): it is not applied again, it
 * bounds the scores for the bounded softmax, as in ga_prefill_attention. */
ga_status ga_prefill_chunk_attention(const ga_attn_desc* desc, int32_t seq_len, const void* q,
                                     const void* k_cache, const void* v_cache, int32_t cache_cap,
                                     const int32_t* cache_lens, const int32_t* chunk_lens,
                                     int32_t max_cache_len, const void* gate, const float* q_norm_w,
                                     const float* k_norm_w, const int32_t* positions, void* workspace,
                                     size_t workspace_bytes, void* out, void* stream);

/* Name of the kernel ga_prefill_chunk_attention runs for this shape:
 * "mirror" (the mirrored prefill kernel with per-sequence key offsets) or
 * "generic"; "unsupported" for a forced kernel that does not serve the
 * shape; "invalid" for a bad descriptor. */
const char* ga_prefill_chunk_kernel(const ga_attn_desc* desc, int32_t seq_len, int32_t cache_cap);

/* ---- decode ------------------------------------------------------------- */

/* Key-chunk length of one decode split (keys per partial result). */
int32_t ga_decode_split_keys(void);

/* Workspace ga_decode needs for caches holding up to max_cache_len tokens:
 * B*H*ceil(max_cache_len/split_keys) partial results of (d + 2) floats. */
size_t ga_decode_workspace_bytes(const ga_attn_desc* desc, int32_t max_cache_len);

/* One decode step for B sequences, each with one new token at position
 * L_b = cache_lens[b]:
 *  q [B,H,d], k_new, v_new [B,G,d]: raw projections of the new token.
 *  gate [B,H,d] | [B,H] | NULL.
 *  k_cache, v_cache [B,cache_cap,G,d]: slots [0,L_b) hold K-hat (already
 *      normed and rotated) and V; they are read as stored. The call writes
 *      the new token's K-hat and V to slot L_b; the caller advances
 *      cache_lens afterwards. The new token attends to the L_b cached keys
 *      and to itself.
 *  cache_lens [B] int32 device array; max_cache_len is a host upper bound of
 *      its values (cache_cap >= max_cache_len + 1). A sequence whose length
 *      is outside [0, max_cache_len] gets NaN outputs and no cache write.
 *  out [B,H*d]. Two kernels: ga_decode_partials then ga_decode_merge. */
ga_status ga_decode(const ga_attn_desc* desc,
                    const void* q, const void* k_new, const void* v_new, const void* gate,
                    const float* q_norm_w, const float* k_norm_w,
                    void* k_cache, void* v_cache, int32_t cache_cap,
                    const int32_t* cache_lens, int32_t max_cache_len,
                    void* workspace, size_t workspace_bytes,
                    void* out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ga_decode
 * without a workspace. The split-K partial results go to a static device
 * array of GA_NOALLOC_SCRATCH_BYTES that each GPU holds, at its own address,
 * from the first call on that device (the calling thread's current device,
 * which must be the stream's) until the process ends; the call allocates
 * nothing. A step whose partials need more than that
 * (ga_decode_workspace_bytes(desc, max_cache_len) > GA_NOALLOC_SCRATCH_BYTES;
 * 48 MiB covers 64 sequences x 8 query heads x 32768 cached tokens at
 * d = 256) returns GA_ERR_WORKSPACE before any launch. Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams,
 * or host threads) race and must be ordered by the caller. Arguments,
 * results and the other errors are those of ga_decode. */
#define GA_NOALLOC_SCRATCH_BYTES (48 * 1024 * 1024)
ga_status ga_decode_noalloc(const ga_attn_desc* desc,
                            const void* q, const void* k_new, const void* v_new, const void* gate,
                            const float* q_norm_w, const float* k_norm_w,
                            void* k_cache, void* v_cache, int32_t cache_cap,
                            const int32_t* cache_lens, int32_t max_cache_len,
                            void* out, void* stream);

/* First stage of ga_decode (one kernel): for every sequence, KV head and key
 * chunk of the cache, the partial softmax state (row max, row sum, unnormed
 * weighted V) of the group's query heads, into the workspace. Reads only
 * slots [0, L_b). */
ga_status ga_decode_partials(const ga_attn_desc* desc, const void* q, const float* q_norm_w,
                             const void* k_cache, const void* v_cache, int32_t cache_cap,
                             const int32_t* cache_lens, int32_t max_cache_len,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Second stage of ga_decode (one kernel): adds the new token's own key and
 * value, merges the partials, applies the gate, writes out and appends the
 * new K-hat and V at slot L_b. */
ga_status ga_decode_merge(const ga_attn_desc* desc, const void* q, const void* k_new,
                          const void* v_new, const void* gate, const float* q_norm_w,
                          const float* k_norm_w, void* k_cache, void* v_cache, int32_t cache_cap,
                          const int32_t* cache_lens, int32_t max_cache_len,
                          const void* workspace, size_t workspace_bytes, void* out, void* stream);

/* ---- backward (training) -------------------------------------------------- */

/* Workspace ga_prefill_backward needs (256-byte aligned): bf16 copies of
 * q-hat, k-hat, the ungated attention output y and its gradient dy, of q-hat,
 * k-hat, v and dy laid out in MFMA operand order (padded to a multiple of 64
 * tokens), fp32 row statistics, fp32 gradients of q-hat and per-head partial
 * gradients of k-hat and v, and 2 x 512 x d floats of weight-gradient
 * partials (about 24 x B*n*H*d bytes for the configs). */
size_t ga_prefill_backward_workspace_bytes(const ga_attn_desc* desc, int32_t seq_len);

/* Backward of ga_prefill: the gradients of sum(dout * out) with respect to
 * every input, for training the layer ("Transformer by Hand · 6. Gated
 * attention", "How the gate is learned": the gate's gradient is
 * dout * y * g(1 - g), then the chain rule through the causal softmax, GQA,
 * RoPE and the RMSNorms of the forward definition above).
 *  q, k, v, gate, q_norm_w, k_norm_w, positions: the forward's inputs.
 *  dout          [B,n,H*d] gradient of the output.
 *  dq [B,n,H,d], dk, dv [B,n,G,d]: written (not accumulated), bf16.
 *  dgate         the gate's shape (required with a gate, unused without).
 *  dq_norm_w, dk_norm_w  [d] float32, written; NULL skips that weight
 *                gradient (also skipped when the weight itself is NULL).
 * Serves bf16, d in {64, 128, 256}, group <= 128, the method's gate
 * (GA_ERR_UNSUPPORTED for gate variants, the output norm, head strides other
 * than dense, fp32). The forward's softmax statistics are recomputed inside
 * the call from q-hat and k-hat, so nothing from the forward call is needed
 * (ga_prefill_backward_lse takes them from ga_prefill_lse instead).
 * Deterministic: no atomics, fixed summation orders. */
ga_status ga_prefill_backward(const ga_attn_desc* desc, int32_t seq_len,
                              const void* q, const void* k, const void* v, const void* gate,
                              const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                              const void* dout, void* dq, void* dk, void* dv, void* dgate,
                              float* dq_norm_w, float* dk_norm_w,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---- training pair with saved row statistics ------------------------------ */

/* Workspace ga_prefill_lse needs (256-byte aligned): bf16 q-hat [B,n,H,d]
 * and k-hat [B,n,G,d], each rounded up to 256 bytes. Depends on its
 * arguments only. */
size_t ga_prefill_lse_workspace_bytes(const ga_attn_desc* desc, int32_t seq_len);

/* Forward for training: out as ga_prefill computes it (no KV cache), plus
 * the statistic of each softmax row that the backward would otherwise
 * recompute: lse[b,i,h] = log2 of sum over keys j <= i of
 * exp2(s_ij * scale * log2 e), s_ij = q_hat_i . k_hat_j (the normalising
 * sum of the causal softmax in "Transformer by Hand · 6. Gated attention",
 * "The formula", kept in log2 form). The probabilities are then
 * P_ij = exp2(s_ij * scale * log2 e - lse_i).
 * k-hat goes to the workspace in bf16 exactly as ga_prefill_backward
 * prepares it; the attention kernel norms and rotates q itself and rounds
 * q-hat to bf16 likewise (where no fused kernel serves the shape, q-hat is
 * prepared in the workspace too). The softmax takes a running row max (not
 * the bounded form of ga_prefill_attention), so lse matches the scores the
 * backward kernels recompute the probabilities from, up to the last bit of
 * an fp32 norm result rounding differently on either side. out can differ
 * from ga_prefill's by bf16 roundings.
 *  q, k, v, gate, q_norm_w, k_norm_w, positions: as for ga_prefill.
 *  workspace     ga_prefill_lse_workspace_bytes bytes, 256-byte aligned.
 *  out           [B,n,H*d] bf16.
 *  lse           [B,n,H] float32, 4-byte aligned, written.
 * Serves the shapes ga_prefill_backward serves (GA_ERR_UNSUPPORTED otherwise). */
ga_status ga_prefill_lse(const ga_attn_desc* desc, int32_t seq_len,
                         const void* q, const void* k, const void* v, const void* gate,
                         const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                         void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream);

/* ga_prefill_backward given the out and lse that ga_prefill_lse wrote for
 * the same inputs: it skips the recomputation of the forward attention.
 * The gate's gradient and the row sums rowsum(dy * y) come from out:
 * dz = dout * out * (1 - g) and rowsum(dout * out), which equal the
 * definitions (dout * y * g(1 - g); dy = dout * g) for out = y * g.
 * Other arguments, the workspace (ga_prefill_backward_workspace_bytes bytes)
 * and the outputs as for ga_prefill_backward. out and lse are read only. */
ga_status ga_prefill_backward_lse(const ga_attn_desc* desc, int32_t seq_len,
                                  const void* q, const void* k, const void* v, const void* gate,
                                  const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                                  const void* out, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv, void* dgate,
                                  float* dq_norm_w, float* dk_norm_w,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---- misc --------------------------------------------------------------- */

const char* ga_status_string(ga_status status);
/* Message for the last failed call on the calling thread ("" if none). */
const char* ga_last_error(void);
/* Which fused kernels serve (dtype, head_dim, rot_dim, group = H/G): bit 0 =
 * the MFMA prefill (bf16, d in {64,128,256}, rot % 16 == 0, group <= 128),
 * bit 1 = the split-K decode (same, group in {1,2,4,8,16}). Shapes without a
 * fused kernel run on the generic one-wave-per-row kernel (any d <= 256,
 * fp32 or bf16); ga_decode_partials/ga_decode_merge need bit 1. The bits
 * are for dense q and gate (see ga_attn_desc for wider head strides). */
int32_t ga_fast_path(int32_t dtype, int32_t head_dim, int32_t rot_dim, int32_t group);
/* ABI version: 6 (ga_attn_desc with head strides, gate variants, the output
 * norm and the kernel-choice fields; k_norm_w in ga_prefill_chunk_attention;
 * the ga_prefill_lse / ga_prefill_backward_lse pair). */
int32_t ga_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GA_H */
