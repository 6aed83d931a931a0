// C ABI: argument validation, dispatch to the fused or generic kernels.
// Every check runs on the host before any launch; nothing is allocated.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "../../include/ga.h"
#include "ga_internal.hpp"

using namespace ga;

namespace {

thread_local char g_last_error[512] = "";

ga_status fail(ga_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

ga_status ok() {
  g_last_error[0] = '\0';
  return GA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int elem_bytes(const ga_attn_desc* d) { return d->dtype == GA_BF16 ? 2 : 4; }

ga_status check_desc(const ga_attn_desc* d) {
  if (!d) return fail(GA_ERR_NULL_ARG, "desc is NULL");
  if (d->dtype != GA_BF16 && d->dtype != GA_F32) return fail(GA_ERR_BAD_DTYPE, "dtype %d out of range", d->dtype);
  if (d->gate_mode < GA_GATE_NONE || d->gate_mode > GA_GATE_ELEMENTWISE)
    return fail(GA_ERR_BAD_DTYPE, "gate_mode %d out of range", d->gate_mode);
  if (d->batch < 0) return fail(GA_ERR_BAD_SHAPE, "batch %d < 0", d->batch);
  if (d->n_q_heads < 1 || d->n_kv_heads < 1) return fail(GA_ERR_BAD_SHAPE, "head counts must be >= 1");
  if (d->n_q_heads % d->n_kv_heads) return fail(GA_ERR_BAD_SHAPE, "n_q_heads %d not a multiple of n_kv_heads %d",
                                                d->n_q_heads, d->n_kv_heads);
  if (d->head_dim < 1) return fail(GA_ERR_BAD_SHAPE, "head_dim %d < 1", d->head_dim);
  if (d->head_dim > 256) return fail(GA_ERR_UNSUPPORTED, "head_dim %d > 256", d->head_dim);
  if (d->rot_dim < 0 || d->rot_dim > d->head_dim || (d->rot_dim & 1))
    return fail(GA_ERR_BAD_SHAPE, "rot_dim %d must be even and in [0, head_dim]", d->rot_dim);
  if (d->rot_dim > 0 && !(d->rope_base > 0.f && isfinite(d->rope_base)))
    return fail(GA_ERR_BAD_SHAPE, "rope_base must be finite and > 0");
  if (!(d->rms_eps >= 0.f && isfinite(d->rms_eps))) return fail(GA_ERR_BAD_SHAPE, "rms_eps must be finite, >= 0");
  if (!(d->softmax_scale >= 0.f && isfinite(d->softmax_scale)))
    return fail(GA_ERR_BAD_SHAPE, "softmax_scale must be finite, >= 0");
  if (d->q_head_stride < 0 || (d->q_head_stride > 0 && d->q_head_stride < d->head_dim))
    return fail(GA_ERR_BAD_SHAPE, "q_head_stride %d must be 0 or >= head_dim %d", d->q_head_stride, d->head_dim);
  const int gw = d->gate_mode == GA_GATE_ELEMENTWISE ? d->head_dim : 1;
  if (d->gate_head_stride < 0 || (d->gate_head_stride > 0 && d->gate_head_stride < gw))
    return fail(GA_ERR_BAD_SHAPE, "gate_head_stride %d must be 0 or >= %d", d->gate_head_stride, gw);
  if (d->gate_act < GA_ACT_SIGMOID || d->gate_act > GA_ACT_IDENTITY)
    return fail(GA_ERR_BAD_DTYPE, "gate_act %d out of range", d->gate_act);
  if (d->gate_combine < GA_COMBINE_MUL || d->gate_combine > GA_COMBINE_ADD)
    return fail(GA_ERR_BAD_DTYPE, "gate_combine %d out of range", d->gate_combine);
  if (d->gate_share < 0 || d->gate_share > (GA_SHARE_HEADS | GA_SHARE_TOKENS))
    return fail(GA_ERR_BAD_DTYPE, "gate_share %d out of range", d->gate_share);
  if (d->kernel < GA_KERNEL_AUTO || d->kernel > GA_KERNEL_GENERIC)
    return fail(GA_ERR_BAD_DTYPE, "kernel %d out of range", d->kernel);
  if (d->bwd_kernel < GA_BWD_AUTO || d->bwd_kernel > GA_BWD_PLAIN)
    return fail(GA_ERR_BAD_DTYPE, "bwd_kernel %d out of range", d->bwd_kernel);
  if (d->out_norm_w) {
    if (!(d->out_norm_eps >= 0.f && isfinite(d->out_norm_eps)))
      return fail(GA_ERR_BAD_SHAPE, "out_norm_eps must be finite, >= 0");
    if (!aligned(d->out_norm_w, 16)) return fail(GA_ERR_MISALIGNED, "out_norm_w is not 16-byte aligned");
  }
  return GA_OK;
}

// Head strides of q and the gate in elements (0 in the descriptor = dense).
long q_stride(const ga_attn_desc* d) { return d->q_head_stride > 0 ? d->q_head_stride : d->head_dim; }
long gate_stride(const ga_attn_desc* d) {
  if (d->gate_head_stride > 0) return d->gate_head_stride;
  return d->gate_mode == GA_GATE_ELEMENTWISE ? d->head_dim : 1;
}

// A gate variant or the output norm: the kernels' extended epilogue.
bool gate_ext(const ga_attn_desc* d) {
  return d->gate_act != GA_ACT_SIGMOID || d->gate_combine != GA_COMBINE_MUL || d->gate_share != 0 ||
         d->out_norm_w != nullptr;
}

// Gate argument of the kernel launchers: the gate mode, or kGateExt.
int gate_arg(const ga_attn_desc* d) { return gate_ext(d) ? kGateExt : d->gate_mode; }

// Offsets of the gate rows (token row t = b*n + i, head h): t * gts + h * ghs.
GateEpi gate_epi(const ga_attn_desc* d) {
  GateEpi ge;
  memset(&ge, 0, sizeof(ge));
  const long s = gate_stride(d);
  const bool heads = d->gate_share & GA_SHARE_HEADS, tokens = d->gate_share & GA_SHARE_TOKENS;
  ge.ghs = heads ? 0 : s;
  ge.gts = tokens ? 0 : (heads ? s : (long)d->n_q_heads * s);
  ge.onorm_w = d->out_norm_w;
  ge.onorm_eps = d->out_norm_eps;
  ge.mode = d->gate_mode;
  ge.act = d->gate_act;
  ge.add = d->gate_combine;
  return ge;
}

// The fused bf16 kernels read q rows and elementwise gate rows in 16-byte
// pieces: their head strides must be multiples of 8 elements.
bool strides_vec_ok(const ga_attn_desc* d) {
  return q_stride(d) % 8 == 0 && (d->gate_mode != GA_GATE_ELEMENTWISE || gate_stride(d) % 8 == 0);
}

float scale_of(const ga_attn_desc* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : (float)(1.0 / sqrt((double)d->head_dim));
}

// Angular frequencies base^(-2t/rot), computed in fp64 on the host.
void fill_inv_freq(const ga_attn_desc* d, double* inv_freq) {
  const int half = d->rot_dim / 2;
  for (int t = 0; t < kMaxHalfRot; ++t)
    inv_freq[t] = (t < half) ? pow((double)d->rope_base, -2.0 * t / (double)d->rot_dim) : 0.0;
}

// Second fused prefill design (mirrored blocks, two key phases, direct-to-LDS
// loads): d in {128, 256}, rot % 16 == 0, group <= 64, and every K/V byte
// offset of one (batch, KV head) within a 31-bit buffer range.
bool prefill_v2_ok(const ga_attn_desc* d, int32_t k_cap, int32_t v_cap) {
  const int grp = d->n_q_heads / d->n_kv_heads;
  const int hd = d->head_dim;
  const long long row = 2LL * d->n_kv_heads * hd;
  // the q prologue keeps every RoPE pair inside one quarter of the row and
  // tables (cos, sin) for the 2 * (64 / grp) tokens of a workgroup
  const int tb = grp <= 64 ? 64 / grp : 0;
  return d->dtype == GA_BF16 && strides_vec_ok(d) && (hd == 128 || hd == 256) && d->rot_dim % 16 == 0 &&
         d->rot_dim <= hd / 4 && grp <= 64 && 2 * tb * (d->rot_dim / 2) <= 2048 && row * k_cap < (1LL << 31) && row * v_cap < (1LL << 31);
}

// The wide kernel: 256 query rows per workgroup, one causal block each,
// heaviest first; it needs enough blocks to balance the triangle (two or more
// per compute unit). RoPE pairs must stay inside one lane: rot/2 % 16 == 0.
bool prefill_wide_ok(const ga_attn_desc* d, int32_t n, int32_t k_cap, int32_t v_cap, bool require_large) {
  const int grp = d->n_q_heads / d->n_kv_heads;
  const int hd = d->head_dim;
  const long long row = 2LL * d->n_kv_heads * hd;
  if (!(d->dtype == GA_BF16 && strides_vec_ok(d) && hd == 128 && d->rot_dim % 32 == 0 && grp <= 256 && row * k_cap < (1LL << 31) &&
        row * v_cap < (1LL << 31)))
    return false;
  const long long tb = 256 / grp;
  const long long blocks = (long long)d->batch * d->n_kv_heads * ((n + tb - 1) / tb);
  return !require_large || blocks >= 512;
}

// Kernel choice for prefill attention: automatic, or the one the descriptor's
// ``kernel`` field names (an error when that kernel does not serve the shape).
enum PrefillKernel { PK_INVALID = -1, PK_AUTO = GA_KERNEL_AUTO, PK_WIDE = GA_KERNEL_WIDE, PK_MIRROR = GA_KERNEL_MIRROR,
                     PK_SIMPLE = GA_KERNEL_SIMPLE, PK_GENERIC = GA_KERNEL_GENERIC };

bool prefill_fast(const ga_attn_desc* d) {
  const int grp = d->n_q_heads / d->n_kv_heads;
  const int hd = d->head_dim;
  return d->dtype == GA_BF16 && strides_vec_ok(d) && (hd == 64 || hd == 128 || hd == 256) && d->rot_dim % 16 == 0 &&
         grp <= 128;
}

// PK_INVALID when a forced kernel does not serve the shape.
PrefillKernel prefill_choice(const ga_attn_desc* d, int32_t n, int32_t k_cap, int32_t v_cap) {
  // (the mirrored kernel numbers output rows (b, token, head) in 32 bits)
  const bool v2 = prefill_v2_ok(d, k_cap, v_cap) && (long long)d->batch * n * d->n_q_heads < (1LL << 31);
  switch (d->kernel) {
    case GA_KERNEL_WIDE: return prefill_wide_ok(d, n, k_cap, v_cap, false) ? PK_WIDE : PK_INVALID;
    case GA_KERNEL_MIRROR: return v2 ? PK_MIRROR : PK_INVALID;
    case GA_KERNEL_SIMPLE: return prefill_fast(d) ? PK_SIMPLE : PK_INVALID;
    case GA_KERNEL_GENERIC: return PK_GENERIC;
    default: break;
  }
  if (prefill_wide_ok(d, n, k_cap, v_cap, true)) return PK_WIDE;
  if (v2) return PK_MIRROR;
  if (prefill_fast(d)) return PK_SIMPLE;
  return PK_GENERIC;
}

// The split decode kernels address one sequence's cache with 32-bit byte
// offsets: cache_cap * G * d * 2 must stay below 2^31 (cache_cap 0: shape only).
bool decode_fast(const ga_attn_desc* d, int32_t cache_cap) {
  const int grp = d->n_q_heads / d->n_kv_heads;
  const int hd = d->head_dim;
  return d->dtype == GA_BF16 && strides_vec_ok(d) && (hd == 64 || hd == 128 || hd == 256) && d->rot_dim % 16 == 0 &&
         (grp == 1 || grp == 2 || grp == 4 || grp == 8 || grp == 16) &&
         (long long)cache_cap * d->n_kv_heads * hd * 2 < (1LL << 31);
}

ga_status check_tensor(const void* p, const char* name, const ga_attn_desc* d, bool required = true) {
  if (!p) return required ? fail(GA_ERR_NULL_ARG, "%s is NULL", name) : GA_OK;
  const size_t a = d->dtype == GA_BF16 ? 16 : 4;
  if (!aligned(p, a)) return fail(GA_ERR_MISALIGNED, "%s is not %zu-byte aligned", name, a);
  return GA_OK;
}

ga_status check_gate(const void* gate, const ga_attn_desc* d) {
  if (d->gate_mode == GA_GATE_NONE) return GA_OK;
  if (!gate) return fail(GA_ERR_NULL_ARG, "gate is NULL but gate_mode is %d", d->gate_mode);
  const size_t a = d->gate_mode == GA_GATE_ELEMENTWISE ? (d->dtype == GA_BF16 ? 16 : 4) : (size_t)elem_bytes(d);
  if (!aligned(gate, a)) return fail(GA_ERR_MISALIGNED, "gate is not %zu-byte aligned", a);
  return GA_OK;
}

// RMSNorm weights: [d] float32, read by the fused kernels in 16-byte pieces.
ga_status check_norm_w(const float* w, const char* name) {
  if (w && !aligned(w, 16)) return fail(GA_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return GA_OK;
}

ga_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t decode_nsplit(int32_t max_len) {
  size_t ns = ((size_t)(max_len > 0 ? max_len : 0) + kDecodeChunk - 1) / kDecodeChunk;
  return ns < 1 ? 1 : ns;
}

// slot_base / row_lens / max_base: a chunk against a cache (NULL, NULL, 0 otherwise)
ga_status prefill_keys_impl(const ga_attn_desc* desc, int32_t n, const void* k, const void* v,
                            const float* k_norm_w, const int32_t* positions, void* k_hat, void* v_out,
                            int32_t kv_cap, hipStream_t stream, const int32_t* slot_base = nullptr,
                            const int32_t* row_lens = nullptr, int32_t max_base = 0) {
  PrepParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.slot_base = slot_base;
  pp.row_lens = row_lens;
  pp.max_base = max_base;
  pp.src = k;
  pp.vsrc = v;
  pp.dst = k_hat;
  pp.vdst = v_out;
  pp.src_bstride = (long)n * desc->n_kv_heads * desc->head_dim;
  pp.vsrc_bstride = pp.src_bstride;
  pp.dst_bstride = (long)kv_cap * desc->n_kv_heads * desc->head_dim;
  pp.vdst_bstride = pp.dst_bstride;
  pp.w = k_norm_w;
  pp.positions = positions;
  pp.B = desc->batch;
  pp.n = n;
  pp.G = desc->n_kv_heads;
  pp.d = desc->head_dim;
  pp.rot = desc->rot_dim;
  pp.eps = desc->rms_eps;
  fill_inv_freq(desc, pp.inv_freq);
  return hip_status(launch_prep_keys(pp, desc->dtype == GA_BF16, stream), "prefill keys launch");
}

// k_norm_w: the weights k_hat was normed with, or null when unknown (then no
// score bound is used). lse: also write each row's log2 log-sum-exp (the
// mirrored and simple kernels only; running-max softmax), or null.
ga_status prefill_attn_impl(const ga_attn_desc* desc, int32_t n, const void* q, const void* k_hat,
                            int32_t k_cap, const void* v, int32_t v_cap, const void* gate,
                            const float* q_norm_w, const float* k_norm_w, const int32_t* positions, void* out,
                            hipStream_t stream, float* lse = nullptr) {
  const int H = desc->n_q_heads, G = desc->n_kv_heads, d = desc->head_dim;
  const int grp = H / G;
  const PrefillKernel choice = prefill_choice(desc, n, k_cap, v_cap);
  const bool wide = choice == PK_WIDE;
  const bool v2 = choice == PK_MIRROR;
  const bool v1 = choice == PK_SIMPLE;
  if (lse && !(v2 || v1)) return fail(GA_ERR_UNSUPPORTED, "row statistics need the mirrored or simple kernel");
  if (wide || v2 || v1) {
    PrefillParams pp;
    memset(&pp, 0, sizeof(pp));
    pp.q = (const uint16_t*)q;
    pp.khat = (const uint16_t*)k_hat;
    pp.v = (const uint16_t*)v;
    pp.gate = (const uint16_t*)gate;
    pp.wq = q_norm_w;
    pp.wk = k_norm_w;
    pp.positions = positions;
    pp.out = (uint16_t*)out;
    pp.lse = lse;
    pp.k_bstride = (long)k_cap * G * d;
    pp.v_bstride = (long)v_cap * G * d;
    pp.qs = q_stride(desc);
    pp.gs = gate_stride(desc);
    pp.ge = gate_epi(desc);
    pp.B = desc->batch;
    pp.n = n;
    pp.H = H;
    pp.G = G;
    pp.grp = grp;
    pp.TB = (wide ? 256 : v2 ? 64 : 128) / grp;  // tokens per block: 256 (wide), 64 (mirror), 128 (simple) rows
    pp.nblk = (n + pp.TB - 1) / pp.TB;
    pp.rot = desc->rot_dim;
    pp.half = desc->rot_dim / 2;
    pp.use_table = ((v2 ? 2 : 1) * pp.TB * pp.half <= 1024) ? 1 : 0;
    pp.eps = desc->rms_eps;
    pp.scale_log2 = scale_of(desc) * 1.4426950408889634f;
    fill_inv_freq(desc, pp.inv_freq);
    if ((long long)pp.B * G * pp.nblk > 0x7fffffffLL) return fail(GA_ERR_UNSUPPORTED, "grid too large");
    if (wide) return hip_status(launch_prefill_wide(pp, d, gate_arg(desc), stream), "prefill attention launch");
    if (v2) return hip_status(launch_prefill_v2(pp, d, gate_arg(desc), stream), "prefill attention launch");
    return hip_status(launch_prefill_mfma(pp, d, gate_arg(desc), stream), "prefill attention launch");
  }
  NaiveParams np;
  memset(&np, 0, sizeof(np));
  np.q = q;
  np.khat = k_hat;
  np.v = v;
  np.gate = gate;
  np.wq = q_norm_w;
  np.positions = positions;
  np.out = out;
  np.k_bstride = (long)k_cap * G * d;
  np.v_bstride = (long)v_cap * G * d;
  np.qs = q_stride(desc);
  np.gs = gate_stride(desc);
  np.ge = gate_epi(desc);
  np.B = desc->batch;
  np.n = n;
  np.H = H;
  np.G = G;
  np.d = d;
  np.rot = desc->rot_dim;
  np.gate_mode = desc->gate_mode;
  np.decode = 0;
  np.eps = desc->rms_eps;
  np.scale = scale_of(desc);
  fill_inv_freq(desc, np.inv_freq);
  return hip_status(launch_naive(np, desc->dtype == GA_BF16, stream), "prefill attention launch");
}

// Kernel of a chunk against a cache: the mirrored kernel (with per-sequence key
// offsets) where it serves the shape, else the generic one; the descriptor
// may force either (an error for a forced mirrored kernel that does not serve it).
PrefillKernel chunk_choice(const ga_attn_desc* d, int32_t n, int32_t cache_cap) {
  const bool mirror = prefill_v2_ok(d, cache_cap, cache_cap) && (long long)d->batch * n * d->n_q_heads < (1LL << 31);
  switch (d->kernel) {
    case GA_KERNEL_AUTO: return mirror ? PK_MIRROR : PK_GENERIC;
    case GA_KERNEL_MIRROR: return mirror ? PK_MIRROR : PK_INVALID;
    case GA_KERNEL_GENERIC: return PK_GENERIC;
    default: return PK_INVALID;
  }
}

// Workspace of the chunk kernels: none today (kept in the ABI for kernels
// that keep partial results).
size_t chunk_ws_bytes(const ga_attn_desc*, int32_t, int32_t, int32_t) { return 0; }

ga_status check_chunk_workspace(const ga_attn_desc* d, int32_t n, int32_t cap, int32_t max_cache_len,
                                const void* workspace, size_t workspace_bytes) {
  const size_t need = chunk_ws_bytes(d, n, cap, max_cache_len);
  if (need == 0) return GA_OK;
  if (!workspace || workspace_bytes < need)
    return fail(GA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 256)) return fail(GA_ERR_MISALIGNED, "workspace is not 256-byte aligned");
  return GA_OK;
}

ga_status check_chunk_common(const ga_attn_desc* desc, int32_t n, const void* k_cache, const void* v_cache,
                             int32_t cache_cap, const int32_t* cache_lens, int32_t max_cache_len) {
  ga_status st;
  if ((st = check_tensor(k_cache, "k_cache", desc)) != GA_OK) return st;
  if ((st = check_tensor(v_cache, "v_cache", desc)) != GA_OK) return st;
  if (!cache_lens) return fail(GA_ERR_NULL_ARG, "cache_lens is NULL");
  if (max_cache_len < 0) return fail(GA_ERR_BAD_SHAPE, "max_cache_len %d < 0", max_cache_len);
  if ((long long)cache_cap < (long long)max_cache_len + n)
    return fail(GA_ERR_BAD_SHAPE, "cache_cap %d < max_cache_len + seq_len (%lld)", cache_cap,
                (long long)max_cache_len + n);
  if ((long long)max_cache_len + n >= (1LL << 30))
    return fail(GA_ERR_UNSUPPORTED, "max_cache_len + seq_len must stay below 2^30");
  return GA_OK;
}

// Compute units of the current device (the chunk kernel's work plan), queried
// once per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

ga_status chunk_attn_impl(const ga_attn_desc* desc, int32_t n, const void* q, const void* k_cache,
                          const void* v_cache, int32_t cap, const int32_t* cache_lens, const int32_t* chunk_lens,
                          int32_t max_cache_len, const void* gate, const float* q_norm_w, const float* k_norm_w,
                          const int32_t* positions, void* workspace, void* out, hipStream_t stream) {
  (void)workspace;
  const int H = desc->n_q_heads, G = desc->n_kv_heads, d = desc->head_dim;
  const int grp = H / G;
  const PrefillKernel choice = chunk_choice(desc, n, cap);
  if (choice == PK_INVALID) return fail(GA_ERR_UNSUPPORTED, "the forced kernel does not serve this chunk shape");
  if (choice == PK_MIRROR) {
    PrefillParams pp;
    memset(&pp, 0, sizeof(pp));
    pp.q = (const uint16_t*)q;
    pp.khat = (const uint16_t*)k_cache;
    pp.v = (const uint16_t*)v_cache;
    pp.gate = (const uint16_t*)gate;
    pp.wq = q_norm_w;
    pp.wk = k_norm_w;
    pp.positions = positions;
    pp.out = (uint16_t*)out;
    pp.key_base = cache_lens;
    pp.row_lens = chunk_lens;
    pp.max_base = max_cache_len;
    pp.ncu = device_cus();
    pp.k_bstride = (long)cap * G * d;
    pp.v_bstride = pp.k_bstride;
    pp.qs = q_stride(desc);
    pp.gs = gate_stride(desc);
    pp.ge = gate_epi(desc);
    pp.B = desc->batch;
    pp.n = n;
    pp.H = H;
    pp.G = G;
    pp.grp = grp;
    pp.TB = 64 / grp;
    pp.nblk = (n + pp.TB - 1) / pp.TB;
    pp.rot = desc->rot_dim;
    pp.half = desc->rot_dim / 2;
    pp.use_table = (2 * pp.TB * pp.half <= 1024) ? 1 : 0;
    pp.eps = desc->rms_eps;
    pp.scale_log2 = scale_of(desc) * 1.4426950408889634f;
    fill_inv_freq(desc, pp.inv_freq);
    if ((long long)pp.B * G * pp.nblk > 0x7fffffffLL) return fail(GA_ERR_UNSUPPORTED, "grid too large");
    return hip_status(launch_prefill_v2(pp, d, gate_arg(desc), stream), "chunk attention launch");
  }
  NaiveParams np;
  memset(&np, 0, sizeof(np));
  np.q = q;
  np.khat = k_cache;
  np.v = v_cache;
  np.gate = gate;
  np.wq = q_norm_w;
  np.positions = positions;
  np.cache_lens = cache_lens;
  np.row_lens = chunk_lens;
  np.out = out;
  np.k_bstride = (long)cap * G * d;
  np.v_bstride = np.k_bstride;
  np.qs = q_stride(desc);
  np.gs = gate_stride(desc);
  np.ge = gate_epi(desc);
  np.B = desc->batch;
  np.n = n;
  np.H = H;
  np.G = G;
  np.d = d;
  np.rot = desc->rot_dim;
  np.gate_mode = desc->gate_mode;
  np.decode = 0;
  np.max_len = max_cache_len;
  np.eps = desc->rms_eps;
  np.scale = scale_of(desc);
  fill_inv_freq(desc, np.inv_freq);
  return hip_status(launch_naive(np, desc->dtype == GA_BF16, stream), "chunk attention launch");
}

ga_status check_decode_common(const ga_attn_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                              int32_t cache_cap, const int32_t* cache_lens, int32_t max_cache_len) {
  ga_status st;
  if ((st = check_tensor(q, "q", desc)) != GA_OK) return st;
  if ((st = check_tensor(k_cache, "k_cache", desc)) != GA_OK) return st;
  if ((st = check_tensor(v_cache, "v_cache", desc)) != GA_OK) return st;
  if (!cache_lens) return fail(GA_ERR_NULL_ARG, "cache_lens is NULL");
  if (max_cache_len < 0) return fail(GA_ERR_BAD_SHAPE, "max_cache_len %d < 0", max_cache_len);
  if ((long long)cache_cap < (long long)max_cache_len + 1)
    return fail(GA_ERR_BAD_SHAPE, "cache_cap %d < max_cache_len + 1 (%d)", cache_cap, max_cache_len + 1);
  return GA_OK;
}

void fill_decode_params(DecodeParams& dp, const ga_attn_desc* desc, const void* q, const void* k_new,
                        const void* v_new, const void* gate, const float* q_norm_w, const float* k_norm_w,
                        const void* k_cache, const void* v_cache, int32_t cache_cap, const int32_t* cache_lens,
                        int32_t max_cache_len, const void* workspace, const void* out) {
  memset(&dp, 0, sizeof(dp));
  const int H = desc->n_q_heads, G = desc->n_kv_heads, d = desc->head_dim;
  dp.q = (const uint16_t*)q;
  dp.k_new = (const uint16_t*)k_new;
  dp.v_new = (const uint16_t*)v_new;
  dp.gate = (const uint16_t*)gate;
  dp.wq = q_norm_w;
  dp.wk = k_norm_w;
  dp.k_cache = (uint16_t*)k_cache;
  dp.v_cache = (uint16_t*)v_cache;
  dp.cache_lens = cache_lens;
  dp.ws = (float*)workspace;
  dp.out = (uint16_t*)out;
  dp.cache_bstride = (long)cache_cap * G * d;
  dp.qs = q_stride(desc);
  dp.gs = gate_stride(desc);
  dp.ge = gate_epi(desc);
  dp.B = desc->batch;
  dp.H = H;
  dp.G = G;
  dp.grp = H / G;
  dp.rot = desc->rot_dim;
  dp.half = desc->rot_dim / 2;
  dp.max_len = max_cache_len;
  dp.nsplit = (int)decode_nsplit(max_cache_len);
  dp.eps = desc->rms_eps;
  dp.scale_log2 = scale_of(desc) * 1.4426950408889634f;
  fill_inv_freq(desc, dp.inv_freq);
}

// Backward workspace: the parts in order, each 256-byte aligned.
struct BwdLayout {
  size_t qh, kh, y, dy, q_rb, q_cb, k_rb, k_cb, v_rb, dy_rb, dy_cb, lse, dsum, dqh, dkp, dvp, wq, wk, total;
  int npad, nwg;
};

constexpr int kBwdNormWorkgroups = 1024;

BwdLayout bwd_layout(const ga_attn_desc* d, int32_t n) {
  BwdLayout L;
  const size_t B = (size_t)d->batch, H = (size_t)d->n_q_heads, G = (size_t)d->n_kv_heads, D = (size_t)d->head_dim;
  L.npad = (int)((n + 63) / 64 * 64);
  L.nwg = kBwdNormWorkgroups;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes, 256);
    return at;
  };
  L.qh = take(B * n * H * D * 2);
  L.kh = take(B * n * G * D * 2);
  L.y = take(B * n * H * D * 2);
  L.dy = take(B * n * H * D * 2);
  L.q_rb = take(B * H * L.npad * D * 2);
  L.q_cb = take(B * H * L.npad * D * 2);
  L.k_rb = take(B * G * L.npad * D * 2);
  L.k_cb = take(B * G * L.npad * D * 2);
  L.v_rb = take(B * G * L.npad * D * 2);
  L.dy_rb = take(B * H * L.npad * D * 2);
  L.dy_cb = take(B * H * L.npad * D * 2);
  L.lse = take(B * n * H * 4);
  L.dsum = take(B * n * H * 4);
  L.dqh = take(B * n * H * D * 4);
  L.dkp = take(B * n * H * D * 4);
  L.dvp = take(B * n * H * D * 4);
  L.wq = take((size_t)L.nwg * D * 4);
  L.wk = take((size_t)L.nwg * D * 4);
  L.total = off;
  return L;
}

// Shapes the backward serves: bf16, d in {64, 128, 256}, group <= 128, the
// method's gate (no variants), dense q and gate.
ga_status check_bwd_desc(const ga_attn_desc* d) {
  const int grp = d->n_q_heads / d->n_kv_heads;
  if (d->dtype != GA_BF16) return fail(GA_ERR_UNSUPPORTED, "the backward pass runs in bf16 only");
  if (!(d->head_dim == 64 || d->head_dim == 128 || d->head_dim == 256))
    return fail(GA_ERR_UNSUPPORTED, "backward: head_dim %d not in {64, 128, 256}", d->head_dim);
  if (grp > 128) return fail(GA_ERR_UNSUPPORTED, "backward: group %d > 128", grp);
  if (gate_ext(d)) return fail(GA_ERR_UNSUPPORTED, "backward: gate variants and the output norm are forward-only");
  if (q_stride(d) != d->head_dim || (d->gate_mode == GA_GATE_ELEMENTWISE && gate_stride(d) != d->head_dim) ||
      (d->gate_mode == GA_GATE_HEADWISE && gate_stride(d) != 1))
    return fail(GA_ERR_UNSUPPORTED, "backward: q and the gate must be dense");
  return GA_OK;
}

}  // namespace

int ga::report(int st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

extern "C" {

size_t ga_prefill_backward_workspace_bytes(const ga_attn_desc* desc, int32_t seq_len) {
  if (check_desc(desc) != GA_OK || seq_len < 0) return 0;
  return bwd_layout(desc, seq_len).total;
}

}  // extern "C"

namespace {

// q-hat and k-hat (bf16, as the MFMA operands of the backward) into qh [B,n,H,d] and kh [B,n,G,d].
ga_status prep_qk_hat(const ga_attn_desc* desc, int32_t n, const void* q, const void* k, const float* q_norm_w,
                      const float* k_norm_w, const int32_t* positions, uint16_t* qh, uint16_t* kh, hipStream_t s) {
  ga_status st;
  if ((st = prefill_keys_impl(desc, n, k, nullptr, k_norm_w, positions, kh, nullptr, n, s)) != GA_OK) return st;
  ga_attn_desc dq_desc = *desc;
  dq_desc.n_kv_heads = desc->n_q_heads;  // the key-preparation kernel over the H query rows of each token
  return prefill_keys_impl(&dq_desc, n, q, nullptr, q_norm_w, positions, qh, nullptr, n, s);
}

// Attention of q-hat against k-hat (no norm and no RoPE left to apply) with
// a running-max softmax, writing the output (gated by ``gate`` under
// gate_mode; y itself for GA_GATE_NONE) and the log2-domain log-sum-exp of
// every row, from the same operands and in the same arithmetic the backward
// kernels recompute the probabilities with.
ga_status attention_stats(const ga_attn_desc* desc, int32_t n, const uint16_t* qh, const uint16_t* kh, const void* v,
                          const void* gate, int gate_mode, void* out, float* lse, hipStream_t s) {
  ga_status st;
  const int B = desc->batch, H = desc->n_q_heads, G = desc->n_kv_heads, D = desc->head_dim;
  PrefillParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.q = qh;
  pp.khat = kh;
  pp.v = (const uint16_t*)v;
  pp.gate = (const uint16_t*)gate;
  pp.out = (uint16_t*)out;
  pp.lse = lse;
  pp.k_bstride = (long)n * G * D;
  pp.v_bstride = pp.k_bstride;
  pp.qs = D;
  pp.gs = gate_mode == GA_GATE_HEADWISE ? 1 : D;
  pp.B = B;
  pp.n = n;
  pp.H = H;
  pp.G = G;
  pp.grp = H / G;
  // the mirrored kernel where it serves the shape, else the simple one
  ga_attn_desc sd = *desc;
  sd.rot_dim = 0;
  sd.gate_mode = gate_mode;
  const bool mirror = prefill_v2_ok(&sd, n, n) && (long long)B * n * H < (1LL << 31);
  pp.TB = (mirror ? 64 : 128) / pp.grp;
  pp.nblk = (n + pp.TB - 1) / pp.TB;
  pp.use_table = 1;
  pp.scale_log2 = scale_of(desc) * 1.4426950408889634f;
  if ((long long)pp.B * G * pp.nblk > 0x7fffffffLL) return fail(GA_ERR_UNSUPPORTED, "grid too large");
  const hipError_t e = mirror ? launch_prefill_v2(pp, D, gate_mode, s) : launch_prefill_mfma(pp, D, gate_mode, s);
  if ((st = hip_status(e, "attention-with-statistics launch")) != GA_OK) return st;
  return GA_OK;
}

// Arguments shared by ga_prefill_backward and ga_prefill_backward_lse.
ga_status check_bwd_args(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k, const void* v,
                         const void* gate, const float* q_norm_w, const float* k_norm_w, const void* dout,
                         void* dq, void* dk, void* dv, void* dgate) {
  ga_status st;
  const char* names[] = {"q", "k", "v", "dout", "dq", "dk", "dv"};
  const void* ptrs[] = {q, k, v, dout, dq, dk, dv};
  for (int i = 0; i < 7; ++i)
    if ((st = check_tensor(ptrs[i], names[i], desc)) != GA_OK) return st;
  if ((st = check_gate(gate, desc)) != GA_OK) return st;
  if (desc->gate_mode != GA_GATE_NONE && (st = check_gate(dgate, desc)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  const long long rows = (long long)desc->batch * seq_len * desc->n_q_heads;
  if (rows >= (1LL << 31)) return fail(GA_ERR_UNSUPPORTED, "backward: B*n*H must stay below 2^31");
  return GA_OK;
}

ga_status check_lse(const float* lse) {
  if (!lse) return fail(GA_ERR_NULL_ARG, "lse is NULL");
  if (!aligned(lse, 4)) return fail(GA_ERR_MISALIGNED, "lse is not 4-byte aligned");
  return GA_OK;
}

// The backward after the argument checks. fwd_out / fwd_lse: the output and
// row statistics of ga_prefill_lse (both NULL: recompute them here).
ga_status backward_impl(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k, const void* v,
                        const void* gate, const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                        const void* fwd_out, const float* fwd_lse, const void* dout, void* dq, void* dk, void* dv,
                        void* dgate, float* dq_norm_w, float* dk_norm_w, void* workspace, size_t workspace_bytes,
                        void* stream) {
  ga_status st;
  const BwdLayout L = bwd_layout(desc, seq_len);
  if (!workspace || workspace_bytes < L.total)
    return fail(GA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? workspace_bytes : 0, L.total);
  if (!aligned(workspace, 256)) return fail(GA_ERR_MISALIGNED, "workspace is not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int B = desc->batch, n = seq_len, H = desc->n_q_heads, G = desc->n_kv_heads, D = desc->head_dim;
  uint16_t* qh = (uint16_t*)(ws + L.qh);
  uint16_t* kh = (uint16_t*)(ws + L.kh);
  uint16_t* y = (uint16_t*)(ws + L.y);
  uint16_t* dyb = (uint16_t*)(ws + L.dy);
  uint16_t* q_rb = (uint16_t*)(ws + L.q_rb);
  uint16_t* q_cb = (uint16_t*)(ws + L.q_cb);
  uint16_t* k_rb = (uint16_t*)(ws + L.k_rb);
  uint16_t* k_cb = (uint16_t*)(ws + L.k_cb);
  uint16_t* v_rb = (uint16_t*)(ws + L.v_rb);
  uint16_t* dy_rb = (uint16_t*)(ws + L.dy_rb);
  uint16_t* dy_cb = (uint16_t*)(ws + L.dy_cb);
  float* lse = (float*)(ws + L.lse);
  float* dsum = (float*)(ws + L.dsum);
  float* dqh = (float*)(ws + L.dqh);
  float* dkp = (float*)(ws + L.dkp);
  float* dvp = (float*)(ws + L.dvp);

  if ((st = prep_qk_hat(desc, n, q, k, q_norm_w, k_norm_w, positions, qh, kh, s)) != GA_OK) return st;
  // the forward's ungated output y and the log-sum-exp of each row, unless the caller kept them
  if (!fwd_lse && (st = attention_stats(desc, n, qh, kh, v, nullptr, GA_GATE_NONE, y, lse, s)) != GA_OK) return st;
  BwdParams bp;
  memset(&bp, 0, sizeof(bp));
  bp.q_rb = q_rb;
  bp.q_cb = q_cb;
  bp.k_rb = k_rb;
  bp.k_cb = k_cb;
  bp.v_rb = v_rb;
  bp.dy_rb = dy_rb;
  bp.dy_cb = dy_cb;
  bp.y = fwd_lse ? (const uint16_t*)fwd_out : y;
  bp.y_is_out = fwd_lse != nullptr;
  bp.dout = (const uint16_t*)dout;
  bp.gate = (const uint16_t*)gate;
  bp.lse = fwd_lse ? fwd_lse : lse;
  bp.dsum = dsum;
  bp.dy_out = dyb;
  bp.dsum_out = dsum;
  bp.dgate = (uint16_t*)dgate;
  bp.dqh = dqh;
  bp.dkp = dkp;
  bp.dvp = dvp;
  bp.B = B;
  bp.n = n;
  bp.npad = L.npad;
  bp.H = H;
  bp.G = G;
  bp.grp = H / G;
  bp.gate_mode = desc->gate_mode;
  bp.plain = desc->bwd_kernel == GA_BWD_PLAIN;
  bp.scale = scale_of(desc);
  bp.scale_log2 = bp.scale * 1.4426950408889634f;
  if ((st = hip_status(launch_bwd_pre(bp, D, s), "backward gate launch")) != GA_OK) return st;
  if ((st = hip_status(launch_bwd_blocks(qh, q_rb, q_cb, B, n, L.npad, H, D, s), "backward operand copies")) != GA_OK ||
      (st = hip_status(launch_bwd_blocks(kh, k_rb, k_cb, B, n, L.npad, G, D, s), "backward operand copies")) != GA_OK ||
      (st = hip_status(launch_bwd_blocks((const uint16_t*)v, v_rb, nullptr, B, n, L.npad, G, D, s),
                       "backward operand copies")) != GA_OK ||
      (st = hip_status(launch_bwd_blocks(dyb, dy_rb, dy_cb, B, n, L.npad, H, D, s), "backward operand copies")) != GA_OK)
    return st;
  if ((st = hip_status(launch_bwd_dq(bp, D, s), "backward dq launch")) != GA_OK) return st;
  if ((st = hip_status(launch_bwd_dkv(bp, D, s), "backward dk/dv launch")) != GA_OK) return st;
  // through RoPE and RMSNorm, q rows then k rows
  for (int which = 0; which < 2; ++which) {
    BwdNormParams np;
    memset(&np, 0, sizeof(np));
    const float* w = which == 0 ? q_norm_w : k_norm_w;
    float* dw = which == 0 ? dq_norm_w : dk_norm_w;
    np.grad = which == 0 ? dqh : dkp;
    np.gsum = which == 0 ? 1 : H / G;
    np.x = (const uint16_t*)(which == 0 ? q : k);
    np.w = w;
    np.positions = positions;
    np.dx = (uint16_t*)(which == 0 ? dq : dk);
    np.wpart = (w && dw) ? (float*)(ws + (which == 0 ? L.wq : L.wk)) : nullptr;
    np.B = B;
    np.n = n;
    np.HX = which == 0 ? H : G;
    np.d = D;
    np.rot = desc->rot_dim;
    np.eps = desc->rms_eps;
    fill_inv_freq(desc, np.inv_freq);
    if ((st = hip_status(launch_bwd_norm_rope(np, L.nwg, s), "backward norm launch")) != GA_OK) return st;
    if (np.wpart && (st = hip_status(launch_bwd_reduce_rows(np.wpart, dw, L.nwg, D, s), "backward reduce")) != GA_OK)
      return st;
  }
  return hip_status(launch_bwd_dv_sum(dvp, (uint16_t*)dv, B, n, H, G, D, s), "backward dv launch");
}

}  // namespace

extern "C" {

ga_status ga_prefill_backward(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k, const void* v,
                              const void* gate, const float* q_norm_w, const float* k_norm_w,
                              const int32_t* positions, const void* dout, void* dq, void* dk, void* dv, void* dgate,
                              float* dq_norm_w, float* dk_norm_w, void* workspace, size_t workspace_bytes,
                              void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if ((st = check_bwd_desc(desc)) != GA_OK) return st;
  if (desc->batch == 0 || seq_len == 0) return ok();
  if ((st = check_bwd_args(desc, seq_len, q, k, v, gate, q_norm_w, k_norm_w, dout, dq, dk, dv, dgate)) != GA_OK)
    return st;
  return backward_impl(desc, seq_len, q, k, v, gate, q_norm_w, k_norm_w, positions, nullptr, nullptr, dout, dq, dk,
                       dv, dgate, dq_norm_w, dk_norm_w, workspace, workspace_bytes, stream);
}

ga_status ga_prefill_backward_lse(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k,
                                  const void* v, const void* gate, const float* q_norm_w, const float* k_norm_w,
                                  const int32_t* positions, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* dgate, float* dq_norm_w, float* dk_norm_w,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if ((st = check_bwd_desc(desc)) != GA_OK) return st;
  if (desc->batch == 0 || seq_len == 0) return ok();
  if ((st = check_bwd_args(desc, seq_len, q, k, v, gate, q_norm_w, k_norm_w, dout, dq, dk, dv, dgate)) != GA_OK)
    return st;
  if ((st = check_tensor(out, "out", desc)) != GA_OK || (st = check_lse(lse)) != GA_OK) return st;
  return backward_impl(desc, seq_len, q, k, v, gate, q_norm_w, k_norm_w, positions, out, lse, dout, dq, dk, dv,
                       dgate, dq_norm_w, dk_norm_w, workspace, workspace_bytes, stream);
}

size_t ga_prefill_lse_workspace_bytes(const ga_attn_desc* desc, int32_t seq_len) {
  if (check_desc(desc) != GA_OK || seq_len < 0) return 0;
  const size_t B = (size_t)desc->batch, H = (size_t)desc->n_q_heads, G = (size_t)desc->n_kv_heads;
  const size_t D = (size_t)desc->head_dim, n = (size_t)seq_len;
  return round_up(B * n * H * D * 2, 256) + round_up(B * n * G * D * 2, 256);
}

ga_status ga_prefill_lse(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k, const void* v,
                         const void* gate, const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                         void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if ((st = check_bwd_desc(desc)) != GA_OK) return st;
  if (desc->batch == 0 || seq_len == 0) return ok();
  const char* names[] = {"q", "k", "v", "out"};
  const void* ptrs[] = {q, k, v, out};
  for (int i = 0; i < 4; ++i)
    if ((st = check_tensor(ptrs[i], names[i], desc)) != GA_OK) return st;
  if ((st = check_gate(gate, desc)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  if ((st = check_lse(lse)) != GA_OK) return st;
  if ((long long)desc->batch * seq_len * desc->n_q_heads >= (1LL << 31))
    return fail(GA_ERR_UNSUPPORTED, "B*n*H must stay below 2^31");
  const size_t need = ga_prefill_lse_workspace_bytes(desc, seq_len);
  if (!workspace || workspace_bytes < need)
    return fail(GA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 256)) return fail(GA_ERR_MISALIGNED, "workspace is not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  uint16_t* qh = (uint16_t*)workspace;
  uint16_t* kh = (uint16_t*)((char*)workspace + round_up((size_t)desc->batch * seq_len * desc->n_q_heads *
                                                             desc->head_dim * 2, 256));
  // The fused kernels norm and rotate q themselves (rounding q-hat to bf16 as
  // the backward's key preparation does, up to the last bit of an fp32
  // result on either side) where one serves the shape with RoPE; otherwise
  // q-hat is prepared here too and the attention runs without norm or RoPE.
  ga_attn_desc fd = *desc;
  fd.kernel = GA_KERNEL_MIRROR;
  if (prefill_choice(&fd, seq_len, seq_len, seq_len) != PK_MIRROR) fd.kernel = GA_KERNEL_SIMPLE;
  if (prefill_choice(&fd, seq_len, seq_len, seq_len) != PK_INVALID) {
    if ((st = prefill_keys_impl(desc, seq_len, k, nullptr, k_norm_w, positions, kh, nullptr, seq_len, s)) != GA_OK)
      return st;
    return prefill_attn_impl(&fd, seq_len, q, kh, seq_len, v, seq_len, gate, q_norm_w, k_norm_w, positions, out, s,
                             lse);
  }
  if ((st = prep_qk_hat(desc, seq_len, q, k, q_norm_w, k_norm_w, positions, qh, kh, s)) != GA_OK) return st;
  return attention_stats(desc, seq_len, qh, kh, v, gate, desc->gate_mode, out, lse, s);
}

const char* ga_prefill_attention_kernel(const ga_attn_desc* desc, int32_t seq_len) {
  if (check_desc(desc) != GA_OK || seq_len < 0) return "invalid";
  switch (prefill_choice(desc, seq_len, seq_len, seq_len)) {
    case PK_WIDE: return "wide";
    case PK_MIRROR: return "mirror";
    case PK_SIMPLE: return "simple";
    case PK_GENERIC: return "generic";
    default: return "unsupported";
  }
}

size_t ga_prefill_workspace_bytes(const ga_attn_desc* desc, int32_t seq_len) {
  if (check_desc(desc) != GA_OK || seq_len < 0) return 0;
  const size_t elems = (size_t)desc->batch * seq_len * desc->n_kv_heads * desc->head_dim;
  return round_up(elems * elem_bytes(desc), 256);
}

ga_status ga_prefill_keys(const ga_attn_desc* desc, int32_t seq_len, const void* k, const void* v,
                          const float* k_norm_w, const int32_t* positions, void* k_hat, void* v_out,
                          int32_t kv_cap, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if (desc->batch == 0 || seq_len == 0) return ok();
  if ((st = check_tensor(k, "k", desc)) != GA_OK) return st;
  if ((st = check_tensor(k_hat, "k_hat", desc)) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  if (v_out) {
    if ((st = check_tensor(v, "v", desc)) != GA_OK) return st;
    if ((st = check_tensor(v_out, "v_out", desc)) != GA_OK) return st;
  }
  if (kv_cap < seq_len) return fail(GA_ERR_BAD_SHAPE, "kv_cap %d < seq_len %d", kv_cap, seq_len);
  return prefill_keys_impl(desc, seq_len, k, v, k_norm_w, positions, k_hat, v_out, kv_cap, (hipStream_t)stream);
}

ga_status ga_prefill_attention(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k_hat,
                               int32_t k_cap, const void* v, int32_t v_cap, const void* gate,
                               const float* q_norm_w, const float* k_norm_w, const int32_t* positions, void* out,
                               void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if (desc->batch == 0 || seq_len == 0) return ok();
  if ((st = check_tensor(q, "q", desc)) != GA_OK) return st;
  if ((st = check_tensor(k_hat, "k_hat", desc)) != GA_OK) return st;
  if ((st = check_tensor(v, "v", desc)) != GA_OK) return st;
  if ((st = check_tensor(out, "out", desc)) != GA_OK) return st;
  if ((st = check_gate(gate, desc)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  if (k_cap < seq_len || v_cap < seq_len)
    return fail(GA_ERR_BAD_SHAPE, "k_cap %d / v_cap %d < seq_len %d", k_cap, v_cap, seq_len);
  if (prefill_choice(desc, seq_len, k_cap, v_cap) == PK_INVALID)
    return fail(GA_ERR_UNSUPPORTED, "the forced kernel %d does not serve this shape", desc->kernel);
  return prefill_attn_impl(desc, seq_len, q, k_hat, k_cap, v, v_cap,
                           desc->gate_mode == GA_GATE_NONE ? nullptr : gate, q_norm_w, k_norm_w, positions, out,
                           (hipStream_t)stream);
}

ga_status ga_prefill(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k, const void* v,
                     const void* gate, const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                     void* k_cache, void* v_cache, int32_t cache_cap, void* workspace, size_t workspace_bytes,
                     void* out, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if (desc->batch == 0 || seq_len == 0) return ok();
  if ((st = check_tensor(q, "q", desc)) != GA_OK) return st;
  if ((st = check_tensor(k, "k", desc)) != GA_OK) return st;
  if ((st = check_tensor(v, "v", desc)) != GA_OK) return st;
  if ((st = check_tensor(out, "out", desc)) != GA_OK) return st;
  if ((st = check_gate(gate, desc)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  void* khat;
  int32_t kcap;
  if (k_cache) {
    if ((st = check_tensor(k_cache, "k_cache", desc)) != GA_OK) return st;
    if ((st = check_tensor(v_cache, "v_cache", desc)) != GA_OK) return st;
    if (cache_cap < seq_len) return fail(GA_ERR_BAD_SHAPE, "cache_cap %d < seq_len %d", cache_cap, seq_len);
    khat = k_cache;
    kcap = cache_cap;
  } else {
    if (v_cache) return fail(GA_ERR_NULL_ARG, "v_cache given without k_cache");
    const size_t need = ga_prefill_workspace_bytes(desc, seq_len);
    if (!workspace || workspace_bytes < need)
      return fail(GA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? workspace_bytes : 0, need);
    if (!aligned(workspace, 16)) return fail(GA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    khat = workspace;
    kcap = seq_len;
  }
  if (prefill_choice(desc, seq_len, kcap, seq_len) == PK_INVALID)
    return fail(GA_ERR_UNSUPPORTED, "the forced kernel %d does not serve this shape", desc->kernel);
  hipStream_t s = (hipStream_t)stream;
  if ((st = prefill_keys_impl(desc, seq_len, k, v, k_norm_w, positions, khat, v_cache, kcap, s)) != GA_OK) return st;
  return prefill_attn_impl(desc, seq_len, q, khat, kcap, v, seq_len,
                           desc->gate_mode == GA_GATE_NONE ? nullptr : gate, q_norm_w, k_norm_w, positions, out, s);
}

const char* ga_prefill_chunk_kernel(const ga_attn_desc* desc, int32_t seq_len, int32_t cache_cap) {
  if (check_desc(desc) != GA_OK || seq_len < 0 || cache_cap < 0) return "invalid";
  switch (chunk_choice(desc, seq_len, cache_cap)) {
    case PK_MIRROR: return "mirror";
    case PK_GENERIC: return "generic";
    default: return "unsupported";
  }
}

size_t ga_prefill_chunk_workspace_bytes(const ga_attn_desc* desc, int32_t seq_len, int32_t cache_cap,
                                        int32_t max_cache_len) {
  if (check_desc(desc) != GA_OK || seq_len < 0 || cache_cap < 0 || max_cache_len < 0) return 0;
  return chunk_ws_bytes(desc, seq_len, cache_cap, max_cache_len);
}

ga_status ga_prefill_chunk_keys(const ga_attn_desc* desc, int32_t seq_len, const void* k, const void* v,
                                const float* k_norm_w, const int32_t* positions, const int32_t* cache_lens,
                                const int32_t* chunk_lens, int32_t max_cache_len, void* k_cache, void* v_cache,
                                int32_t cache_cap, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if (desc->batch == 0 || seq_len == 0) return ok();
  if ((st = check_tensor(k, "k", desc)) != GA_OK) return st;
  if ((st = check_tensor(v, "v", desc)) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  if ((st = check_chunk_common(desc, seq_len, k_cache, v_cache, cache_cap, cache_lens, max_cache_len)) != GA_OK)
    return st;
  return prefill_keys_impl(desc, seq_len, k, v, k_norm_w, positions, k_cache, v_cache, cache_cap,
                           (hipStream_t)stream, cache_lens, chunk_lens, max_cache_len);
}

ga_status ga_prefill_chunk_attention(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k_cache,
                                     const void* v_cache, int32_t cache_cap, const int32_t* cache_lens,
                                     const int32_t* chunk_lens, int32_t max_cache_len, const void* gate,
                                     const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                                     void* workspace, size_t workspace_bytes, void* out, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if (desc->batch == 0 || seq_len == 0) return ok();
  if ((st = check_tensor(q, "q", desc)) != GA_OK) return st;
  if ((st = check_tensor(out, "out", desc)) != GA_OK) return st;
  if ((st = check_gate(gate, desc)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  if ((st = check_chunk_common(desc, seq_len, k_cache, v_cache, cache_cap, cache_lens, max_cache_len)) != GA_OK)
    return st;
  if ((st = check_chunk_workspace(desc, seq_len, cache_cap, max_cache_len, workspace, workspace_bytes)) != GA_OK)
    return st;
  if (chunk_choice(desc, seq_len, cache_cap) == PK_INVALID)
    return fail(GA_ERR_UNSUPPORTED, "the forced kernel %d does not serve this chunk shape", desc->kernel);
  return chunk_attn_impl(desc, seq_len, q, k_cache, v_cache, cache_cap, cache_lens, chunk_lens, max_cache_len,
                         desc->gate_mode == GA_GATE_NONE ? nullptr : gate, q_norm_w, k_norm_w, positions, workspace,
                         out, (hipStream_t)stream);
}

ga_status ga_prefill_chunk(const ga_attn_desc* desc, int32_t seq_len, const void* q, const void* k, const void* v,
                           const void* gate, const float* q_norm_w, const float* k_norm_w, const int32_t* positions,
                           void* k_cache, void* v_cache, int32_t cache_cap, const int32_t* cache_lens,
                           const int32_t* chunk_lens, int32_t max_cache_len, void* workspace,
                           size_t workspace_bytes, void* out, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (seq_len < 0) return fail(GA_ERR_BAD_SHAPE, "seq_len %d < 0", seq_len);
  if (desc->batch == 0 || seq_len == 0) return ok();
  if ((st = check_tensor(q, "q", desc)) != GA_OK) return st;
  if ((st = check_tensor(k, "k", desc)) != GA_OK) return st;
  if ((st = check_tensor(v, "v", desc)) != GA_OK) return st;
  if ((st = check_tensor(out, "out", desc)) != GA_OK) return st;
  if ((st = check_gate(gate, desc)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  if ((st = check_chunk_common(desc, seq_len, k_cache, v_cache, cache_cap, cache_lens, max_cache_len)) != GA_OK)
    return st;
  if ((st = check_chunk_workspace(desc, seq_len, cache_cap, max_cache_len, workspace, workspace_bytes)) != GA_OK)
    return st;
  if (chunk_choice(desc, seq_len, cache_cap) == PK_INVALID)
    return fail(GA_ERR_UNSUPPORTED, "the forced kernel %d does not serve this chunk shape", desc->kernel);
  hipStream_t s = (hipStream_t)stream;
  if ((st = prefill_keys_impl(desc, seq_len, k, v, k_norm_w, positions, k_cache, v_cache, cache_cap, s, cache_lens,
                              chunk_lens, max_cache_len)) != GA_OK)
    return st;
  return chunk_attn_impl(desc, seq_len, q, k_cache, v_cache, cache_cap, cache_lens, chunk_lens, max_cache_len,
                         desc->gate_mode == GA_GATE_NONE ? nullptr : gate, q_norm_w, k_norm_w, positions, workspace,
                         out, s);
}

int32_t ga_decode_split_keys(void) { return kDecodeChunk; }

size_t ga_decode_workspace_bytes(const ga_attn_desc* desc, int32_t max_cache_len) {
  if (check_desc(desc) != GA_OK || max_cache_len < 0) return 0;
  const size_t per = (size_t)desc->batch * desc->n_q_heads * decode_nsplit(max_cache_len);
  return round_up(per * (desc->head_dim + 2) * sizeof(float), 256);
}

ga_status ga_decode_partials(const ga_attn_desc* desc, const void* q, const float* q_norm_w, const void* k_cache,
                             const void* v_cache, int32_t cache_cap, const int32_t* cache_lens,
                             int32_t max_cache_len, void* workspace, size_t workspace_bytes, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (desc->batch == 0) return ok();
  if (!decode_fast(desc, cache_cap))
    return fail(GA_ERR_UNSUPPORTED, "decode stages need the fused path (bf16, d in {64,128,256}, rot %% 16 == 0, "
                                    "group in {1,2,4,8,16}, cache_cap * G * d * 2 < 2^31)");
  if ((st = check_decode_common(desc, q, k_cache, v_cache, cache_cap, cache_lens, max_cache_len)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  const size_t need = ga_decode_workspace_bytes(desc, max_cache_len);
  if (!workspace || workspace_bytes < need)
    return fail(GA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 16)) return fail(GA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  DecodeParams dp;
  fill_decode_params(dp, desc, q, nullptr, nullptr, nullptr, q_norm_w, nullptr, k_cache, v_cache, cache_cap,
                     cache_lens, max_cache_len, workspace, nullptr);
  return hip_status(launch_decode_partials(dp, desc->head_dim, (hipStream_t)stream), "decode partials launch");
}

ga_status ga_decode_merge(const ga_attn_desc* desc, const void* q, const void* k_new, const void* v_new,
                          const void* gate, const float* q_norm_w, const float* k_norm_w, void* k_cache,
                          void* v_cache, int32_t cache_cap, const int32_t* cache_lens, int32_t max_cache_len,
                          const void* workspace, size_t workspace_bytes, void* out, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (desc->batch == 0) return ok();
  if (!decode_fast(desc, cache_cap))
    return fail(GA_ERR_UNSUPPORTED, "decode stages need the fused path (bf16, d in {64,128,256}, rot %% 16 == 0, "
                                    "group in {1,2,4,8,16}, cache_cap * G * d * 2 < 2^31)");
  if ((st = check_decode_common(desc, q, k_cache, v_cache, cache_cap, cache_lens, max_cache_len)) != GA_OK) return st;
  if ((st = check_tensor(k_new, "k_new", desc)) != GA_OK) return st;
  if ((st = check_tensor(v_new, "v_new", desc)) != GA_OK) return st;
  if ((st = check_tensor(out, "out", desc)) != GA_OK) return st;
  if ((st = check_gate(gate, desc)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  const size_t need = ga_decode_workspace_bytes(desc, max_cache_len);
  if (!workspace || workspace_bytes < need)
    return fail(GA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 16)) return fail(GA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  DecodeParams dp;
  fill_decode_params(dp, desc, q, k_new, v_new, desc->gate_mode == GA_GATE_NONE ? nullptr : gate, q_norm_w,
                     k_norm_w, k_cache, v_cache, cache_cap, cache_lens, max_cache_len, workspace, out);
  return hip_status(launch_decode_merge(dp, desc->head_dim, gate_arg(desc), (hipStream_t)stream),
                    "decode merge launch");
}

ga_status ga_decode(const ga_attn_desc* desc, const void* q, const void* k_new, const void* v_new, const void* gate,
                    const float* q_norm_w, const float* k_norm_w, void* k_cache, void* v_cache, int32_t cache_cap,
                    const int32_t* cache_lens, int32_t max_cache_len, void* workspace, size_t workspace_bytes,
                    void* out, void* stream) {
  ga_status st;
  if ((st = check_desc(desc)) != GA_OK) return st;
  if (desc->batch == 0) return ok();
  if ((st = check_decode_common(desc, q, k_cache, v_cache, cache_cap, cache_lens, max_cache_len)) != GA_OK) return st;
  if ((st = check_tensor(k_new, "k_new", desc)) != GA_OK) return st;
  if ((st = check_tensor(v_new, "v_new", desc)) != GA_OK) return st;
  if ((st = check_tensor(out, "out", desc)) != GA_OK) return st;
  if ((st = check_gate(gate, desc)) != GA_OK) return st;
  if ((st = check_norm_w(q_norm_w, "q_norm_w")) != GA_OK) return st;
  if ((st = check_norm_w(k_norm_w, "k_norm_w")) != GA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (decode_fast(desc, cache_cap)) {
    if ((st = ga_decode_partials(desc, q, q_norm_w, k_cache, v_cache, cache_cap, cache_lens, max_cache_len,
                                 workspace, workspace_bytes, stream)) != GA_OK)
      return st;
    return ga_decode_merge(desc, q, k_new, v_new, gate, q_norm_w, k_norm_w, k_cache, v_cache, cache_cap, cache_lens,
                           max_cache_len, workspace, workspace_bytes, out, stream);
  }
  NaiveParams np;
  memset(&np, 0, sizeof(np));
  const int G = desc->n_kv_heads, d = desc->head_dim;
  np.q = q;
  np.khat = k_cache;
  np.v = v_cache;
  np.gate = desc->gate_mode == GA_GATE_NONE ? nullptr : gate;
  np.wq = q_norm_w;
  np.wk = k_norm_w;
  np.cache_lens = cache_lens;
  np.k_new = k_new;
  np.v_new = v_new;
  np.k_cache_out = k_cache;
  np.v_cache_out = v_cache;
  np.out = out;
  np.k_bstride = (long)cache_cap * G * d;
  np.v_bstride = np.k_bstride;
  np.qs = q_stride(desc);
  np.gs = gate_stride(desc);
  np.ge = gate_epi(desc);
  np.B = desc->batch;
  np.n = 1;
  np.H = desc->n_q_heads;
  np.G = G;
  np.d = d;
  np.rot = desc->rot_dim;
  np.gate_mode = desc->gate_mode;
  np.decode = 1;
  np.max_len = max_cache_len;
  np.eps = desc->rms_eps;
  np.scale = scale_of(desc);
  fill_inv_freq(desc, np.inv_freq);
  return hip_status(launch_naive(np, desc->dtype == GA_BF16, s), "decode launch");
}

const char* ga_status_string(ga_status status) {
  switch (status) {
    case GA_OK: return "GA_OK";
    case GA_ERR_NULL_ARG: return "GA_ERR_NULL_ARG";
    case GA_ERR_BAD_SHAPE: return "GA_ERR_BAD_SHAPE";
    case GA_ERR_BAD_DTYPE: return "GA_ERR_BAD_DTYPE";
    case GA_ERR_UNSUPPORTED: return "GA_ERR_UNSUPPORTED";
    case GA_ERR_MISALIGNED: return "GA_ERR_MISALIGNED";
    case GA_ERR_WORKSPACE: return "GA_ERR_WORKSPACE";
    case GA_ERR_HIP: return "GA_ERR_HIP";
    default: return "GA_ERR_UNKNOWN";
  }
}

const char* ga_last_error(void) { return g_last_error; }

int32_t ga_fast_path(int32_t dtype, int32_t head_dim, int32_t rot_dim, int32_t group) {
  ga_attn_desc d;
  memset(&d, 0, sizeof(d));
  d.dtype = dtype;
  d.head_dim = head_dim;
  d.rot_dim = rot_dim;
  d.n_kv_heads = 1;
  d.n_q_heads = group > 0 ? group : 1;
  return (prefill_fast(&d) ? 1 : 0) | (decode_fast(&d, 0) ? 2 : 0);
}

int32_t ga_version(void) { return 6; }

}  // extern "C"
