// Kernel parameter blocks and launchers shared between the kernel files and
// the C ABI layer (ga_api.hip). Host-side declarations only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

constexpr int kMaxHalfRot = 128;  // rot_dim <= 256

// Gate variants and the per-head output norm. The fused kernels read these
// only in their extended-epilogue instantiation (gate template argument
// kGateExt); their default instantiations apply y * sigmoid(z) as before.
struct GateEpi {
  long gts, ghs;          // logits of (token row t = b*n + i, head h) start at t * gts + h * ghs
  const float* onorm_w;   // [d]: per-head RMSNorm of the attention output (before the gate), or null
  float onorm_eps;
  int mode;               // 0 none, 1 headwise, 2 elementwise
  int act;                // 0 sigmoid(z), 1 0.5 + 0.5 sigmoid(z), 2 z sigmoid(z), 3 z
  int add;                // 0: y * act(z); 1: y + act(z)
};
constexpr int kGateExt = 3;

// K-hat = RoPE(RMSNorm(k)) for [B,n,G,d] rows; optional copy of v.
struct PrepParams {
  const void* src;     // k rows, [B, *, G, d] with batch stride src_bstride
  const void* vsrc;    // v rows or null
  void* dst;           // K-hat rows
  void* vdst;          // copy of v, or null
  long src_bstride, vsrc_bstride, dst_bstride, vdst_bstride;  // elements per batch
  const float* w;      // [d] or null
  const int* positions;  // [B, n] or null (= slot index)
  // Chunk against a cache (both null otherwise): row i of sequence b goes to
  // slot slot_base[b] + i, and only rows i < row_lens[b] are written.
  const int* slot_base;  // [B] or null (= 0)
  const int* row_lens;   // [B] or null (= n)
  int max_base;          // slot_base values outside [0, max_base] skip the sequence
  int B, n, G, d, rot;
  float eps;
  double inv_freq[kMaxHalfRot];
};

// Fused MFMA prefill (bf16).
struct PrefillParams {
  const uint16_t* q;
  const uint16_t* khat;
  const uint16_t* v;
  const uint16_t* gate;
  const float* wq;
  // k-norm weights that k_hat was normed with (null: unknown). With wq they
  // bound every score, and the kernels drop the running row max.
  const float* wk;
  const int* positions;
  uint16_t* out;
  // Chunk against a cache (mirrored kernel only; both null otherwise): the
  // n query rows of sequence b are tokens key_base[b] + i of it, of which
  // rows i < row_lens[b] are real; row i sees keys [0, key_base[b] + i].
  const int* key_base;  // [B] or null (= 0)
  const int* row_lens;  // [B] or null (= n)
  int max_base;         // key_base values outside [0, max_base] skip the sequence
  int ncu;              // compute units of the device (chunk work plan)
  long k_bstride, v_bstride;
  // elements between the rows of consecutive heads of q and of the gate (a
  // token's rows follow each other: token stride = H * stride)
  long qs, gs;
  GateEpi ge;
  int B, n, H, G, grp, TB, nblk, rot, half, use_table;
  float eps, scale_log2;
  // log2-domain log-sum-exp of each output row (b, token, head), for the
  // backward pass (simple and mirrored kernels, running-max softmax, the
  // method's gate only); null otherwise
  float* lse;
  double inv_freq[kMaxHalfRot];
};

// Generic (any d <= 256) attention, one wave per query row. Used for fp32 and
// for shapes without a fused kernel. For decode, rows attend to a cache plus
// the new token.
struct NaiveParams {
  const void* q;        // prefill [B,n,H,d]; decode [B,H,d]
  const void* khat;     // prepared keys [B, kcap, G, d] (prefill or cache)
  const void* v;        // values [B, vcap, G, d]
  const void* gate;
  const float* wq;
  const float* wk;      // decode: k_new norm weight
  const int* positions; // prefill positions or null
  const int* cache_lens;  // decode: cached keys; chunked prefill: keys before the chunk (or null)
  const int* row_lens;    // chunked prefill: real rows per sequence (or null = n)
  const void* k_new;    // decode only
  const void* v_new;    // decode only
  void* k_cache_out;    // decode: slot L written (k_cache base)
  void* v_cache_out;
  void* out;
  long k_bstride, v_bstride;
  long qs, gs;          // head strides of q and the gate (elements)
  GateEpi ge;           // gate form and offsets (this kernel always reads them)
  int B, n, H, G, d, rot, gate_mode, decode, max_len;
  float eps, scale;
  double inv_freq[kMaxHalfRot];
};

// Fused decode (bf16): split kernel + merge kernel.
struct DecodeParams {
  const uint16_t* q;        // [B,H,D]
  const uint16_t* k_new;    // [B,G,D]
  const uint16_t* v_new;
  const uint16_t* gate;
  const float* wq;
  const float* wk;
  uint16_t* k_cache;        // [B,cap,G,D]
  uint16_t* v_cache;
  const int* cache_lens;
  float* ws;                // partials
  uint16_t* out;            // [B,H*D]
  long cache_bstride;       // cap*G*D
  long qs, gs;              // head strides of q and the gate (elements)
  GateEpi ge;
  int B, H, G, grp, rot, half, max_len, nsplit;
  float eps, scale_log2;
  double inv_freq[kMaxHalfRot];
};

constexpr int kDecodeChunk = 768;  // keys per decode split

// Backward of the prefill (bf16). Row-major workspace copies: y [B,n,H,d]
// (ungated attention output; or, with y_is_out, the caller's gated output), dy [B,n,H,d] (gradient of y); lse, dsum
// [B,n,H] fp32 (log2-domain log-sum-exp of each score row; rowsum(dy * y)).
// MFMA-operand copies (bf16, zero past n, npad tokens): row-blocked
// ("rb": 32 tokens x 16 dims per 1 KiB piece, lane l holding token l%32,
// dims 8(l/32)..+8) of q-hat, dy [B,H] and k-hat, v [B,G]; column-blocked
// ("cb": 32 dims x 16 tokens per piece, lane l holding dim l%32, tokens
// 4(l/32)+0..3 and 8+4(l/32)+0..3) of q-hat, dy [B,H] and k-hat [B,G].
// Outputs: dqh [B,n,H,d] fp32; per-head partial dk-hat and dv, dkp and dvp
// [B,n,H,d] fp32 (summed over each group's heads afterwards).
struct BwdParams {
  const uint16_t* q_rb;
  const uint16_t* q_cb;
  const uint16_t* k_rb;
  const uint16_t* k_cb;
  const uint16_t* v_rb;
  const uint16_t* dy_rb;
  const uint16_t* dy_cb;
  const uint16_t* y;
  const uint16_t* dout;
  const uint16_t* gate;
  const float* lse;
  const float* dsum;
  uint16_t* dy_out;     // pre kernel: dy
  float* dsum_out;      // pre kernel: dsum
  uint16_t* dgate;      // pre kernel: gradient of the gate logits (or null)
  float* dqh;
  float* dkp;
  float* dvp;
  int B, n, npad, H, G, grp, gate_mode;
  int plain;            // 1: the register-operand dq and dK/dV kernels for every shape
  int y_is_out;         // pre kernel: y holds the forward's gated output (see bwd_pre_kernel)
  float scale, scale_log2;
};

// Gradient of x through n = RoPE(RMSNorm(x, w)) for rows [B, n, HX, d]:
// grad (fp32 gradient of n) -> dx (bf16); per-workgroup partial sums of the
// weight gradient in wpart [gridDim.x][d] when w is not null. The gradient
// of row (t, x) is the sum of gsum rows (t, x*gsum + 0..gsum-1) of grad
// [B, n, HX*gsum, d] (the per-head partials of a KV head; gsum = 1 for q).
struct BwdNormParams {
  const float* grad;
  int gsum;
  const uint16_t* x;
  const float* w;
  const int* positions;
  uint16_t* dx;
  float* wpart;
  int B, n, HX, d, rot;
  float eps;
  double inv_freq[kMaxHalfRot];
};

hipError_t launch_bwd_pre(const BwdParams& p, int D, hipStream_t s);
// MFMA-operand copies of src [B, n, HX, D]: row-blocked and/or column-blocked (null skips)
hipError_t launch_bwd_blocks(const uint16_t* src, uint16_t* rb, uint16_t* cb, int B, int n, int npad, int HX, int D,
                             hipStream_t s);
// dv [B,n,G,D] bf16 = sum of the group's per-head partials dvp [B,n,H,D]
hipError_t launch_bwd_dv_sum(const float* dvp, uint16_t* dv, int B, int n, int H, int G, int D, hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, int D, hipStream_t s);
hipError_t launch_bwd_dkv(const BwdParams& p, int D, hipStream_t s);
hipError_t launch_bwd_norm_rope(const BwdNormParams& p, int nwg, hipStream_t s);
hipError_t launch_bwd_reduce_rows(const float* part, float* out, int nrows, int d, hipStream_t s);

// Records a message for ga_last_error() on the calling thread and returns st
// (the status codes of include/ga.h).
int report(int st, const char* fmt, ...);

hipError_t launch_prep_keys(const PrepParams& p, int is_bf16, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillParams& p, int D, int gate_mode, hipStream_t s);
hipError_t launch_prefill_v2(const PrefillParams& p, int D, int gate_mode, hipStream_t s);
hipError_t launch_prefill_wide(const PrefillParams& p, int D, int gate_mode, hipStream_t s);
hipError_t launch_naive(const NaiveParams& p, int is_bf16, hipStream_t s);
hipError_t launch_decode_partials(const DecodeParams& p, int D, hipStream_t s);
hipError_t launch_decode_merge(const DecodeParams& p, int D, int gate_mode, hipStream_t s);

}  // namespace ga
