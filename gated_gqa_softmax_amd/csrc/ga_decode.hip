// Split-K decode for gfx950 (bf16 cache, fp32 accumulation).
//
// One decode step: a new query token at position L attends to the L cached
// keys (already normed and rotated) and to its own key, and mixes the cached
// values and its own value ("多头注意力与 GQA", section "标准多头注意力（MHA）":
// the new query is dotted with every cached key; Q is never cached). The
// KV-cache stream dominates ("多头注意力与 GQA", "工程要点": the cache, not the
// weights, fills memory and sets decode latency), so the kernels are built
// around reading each cached byte once at full HBM rate:
//
//  * decode_partials_kernel: one workgroup per (sequence, KV head, chunk of
//    kDecodeChunk keys). All query heads of the GQA group are processed
//    together, so every K/V byte is read once per group. Scores come from
//    v_mfma_f32_16x16x32_bf16 with K rows loaded straight from HBM into the A
//    operand (16-byte loads, 64 contiguous bytes per row per instruction);
//    the chunk's softmax is exact within the chunk (max first, then exp);
//    the value mix streams V rows with 16-byte loads (each lane owns 8 dims)
//    and reduces across wavefronts in LDS. Output: per (head, chunk) the
//    chunk max m, sum l and unnormalised o[d], in the workspace.
//  * decode_merge_kernel: per (sequence, KV head), adds the new token's own
//    score, merges the chunks (rescaling by 2^(m_c - M)), applies the sigmoid
//    gate and stores bf16 output; appends the new K-hat and V to slot L.
//    Chunks never read slot L, so the append cannot race with them.
#include "ga_common.hpp"
#include "ga_internal.hpp"

namespace ga {

template <int D, int GRP>
__global__ __launch_bounds__(256) void decode_partials_kernel(const DecodeParams p) {
  constexpr int C = kDecodeChunk;
  constexpr int SQ = D + 8;
  constexpr int LPR = D / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  uint16_t* Qs = (uint16_t*)dyn_smem;                 // [16][SQ] bf16 q-hat (rows >= GRP are 0)
  float* Ssc = (float*)(dyn_smem + 16 * SQ * 2);      // [C][GRP] scores, then probabilities
  float* Red = Ssc;                                   // reused: [4][GRP][D] wave partials

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int split = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / p.G, g = bg % p.G;
  int L = p.cache_lens[b];
  if (L < 0 || L > p.max_len) L = 0;
  const int start = split * C;
  if (start >= L) return;
  const int nk = min(C, L - start);

  // q-hat of the group's heads at position L (same rounding as prefill: bf16)
  for (int idx = tid; idx < 16 * LPR; idx += 256) {
    const int r = idx / LPR, c = idx % LPR;
    u32x4_t raw = {0, 0, 0, 0};
    if (r < GRP) raw = *(const u32x4_t*)(p.q + ((long)b * p.H + g * GRP + r) * D + c * 8);
    float x[8];
    unpack8(raw, x);
    norm_rope_chunk<D>(x, c, p.wq, p.eps, p.rot, L, p.inv_freq, nullptr);
    *(u32x4_t*)(Qs + r * SQ + c * 8) = pack8(x);
  }
  __syncthreads();

  // ---- scores: S^T[key][head] = K-hat . q-hat, 16 keys per MFMA group -------
  const int l16 = lane & 15, q4 = lane >> 4;
  bf16x8_t qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qf[c] = *(const bf16x8_t*)(Qs + l16 * SQ + c * 32 + q4 * 8);
  const uint16_t* Kc = p.k_cache + (long)b * p.cache_bstride + (long)g * D;
  const uint16_t* Vc = p.v_cache + (long)b * p.cache_bstride + (long)g * D;
  const long row = (long)p.G * D;
  const int ngroups = (nk + 15) / 16;
  for (int gi = w; gi < ngroups; gi += 4) {
    const int key = start + gi * 16 + l16;
    const bool kval = key < start + nk;
    u32x4_t kr[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      kr[c] = kval ? *(const u32x4_t*)(Kc + key * row + c * 32 + q4 * 8) : u32x4_t{0, 0, 0, 0};
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[c]), qf[c], acc, 0, 0, 0);
    // acc[i]: head l16, key gi*16 + 4*q4 + i
    if (l16 < GRP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kl = gi * 16 + q4 * 4 + i;
        if (kl < C) Ssc[kl * GRP + l16] = (kl < nk) ? acc[i] * p.scale_log2 : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- chunk softmax per head (exact within the chunk) ----------------------
  float* ws_o = p.ws;
  float* ws_ml = p.ws + (long)p.B * p.H * p.nsplit * D;
  for (int h = w; h < GRP; h += 4) {
    float mx = -INFINITY;
    for (int k = lane; k < nk; k += 64) mx = fmaxf(mx, Ssc[k * GRP + h]);
    mx = max_xor<64>(mx);
    float sm = 0.f;
    for (int k = lane; k < nk; k += 64) {
      const float e = __builtin_amdgcn_exp2f(Ssc[k * GRP + h] - mx);
      Ssc[k * GRP + h] = e;
      sm += e;
    }
    sm = sum_xor<64>(sm);
    if (lane == 0) {
      const long idx = ((long)b * p.H + g * GRP + h) * p.nsplit + split;
      ws_ml[idx * 2 + 0] = mx;
      ws_ml[idx * 2 + 1] = sm;
    }
  }
  __syncthreads();

  // ---- value mix: lane owns 8 dims of one key slot ---------------------------
  constexpr int KPW = 64 / LPR;  // key slots per wave
  const int dc = lane % LPR, ks = lane / LPR;
  float acc[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  constexpr int STEP = 4 * KPW;
  constexpr int UNROLL = 4;
  for (int k0 = w * KPW + ks; k0 < nk; k0 += STEP * UNROLL) {
    u32x4_t vr[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = k0 + u * STEP;
      vr[u] = (k < nk) ? *(const u32x4_t*)(Vc + (long)(start + k) * row + dc * 8) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = k0 + u * STEP;
      if (k < nk) {
        float v[8];
        unpack8(vr[u], v);
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          const float pw = Ssc[k * GRP + h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] += pw * v[e];
        }
      }
    }
  }
  // reduce over key slots inside the wave
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], m, 64);
  __syncthreads();  // Ssc no longer needed: reuse as Red
  if (ks == 0) {
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) Red[(w * GRP + h) * D + dc * 8 + e] = acc[h][e];
  }
  __syncthreads();
  for (int idx = tid; idx < GRP * D; idx += 256) {
    const int h = idx / D, e = idx % D;
    const float s = Red[(0 * GRP + h) * D + e] + Red[(1 * GRP + h) * D + e] + Red[(2 * GRP + h) * D + e] +
                    Red[(3 * GRP + h) * D + e];
    ws_o[(((long)b * p.H + g * GRP + h) * p.nsplit + split) * D + e] = s;
  }
}

template <int D, int GATE>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeParams p) {
  constexpr int LPR = D / 8;
  constexpr int SPLITS_PER_PASS = 256;
  __shared__ float qk[17][D];       // rows 0..grp-1: q-hat (bf16-rounded); row 16: k-hat new
  __shared__ float snew[16];
  __shared__ float mtot[16], ltot[16];
  __shared__ float wts[16][SPLITS_PER_PASS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bg = blockIdx.x;
  const int b = bg / p.G, g = bg % p.G;
  const int grp = p.grp;
  const int L = p.cache_lens[b];
  uint16_t* out = p.out + ((long)b * p.H + g * grp) * D;
  if (L < 0 || L > p.max_len) {
    for (int idx = tid; idx < grp * D; idx += 256) out[idx] = 0x7fc0;  // NaN
    return;
  }

  // q-hat rows and the new key row: norm + rope at position L, rounded to bf16
  for (int idx = tid; idx < 17 * LPR; idx += 256) {
    const int r = idx / LPR, c = idx % LPR;
    const bool is_k = (r == 16);
    u32x4_t raw = {0, 0, 0, 0};
    if (is_k) raw = *(const u32x4_t*)(p.k_new + ((long)b * p.G + g) * D + c * 8);
    else if (r < grp) raw = *(const u32x4_t*)(p.q + ((long)b * p.H + g * grp + r) * D + c * 8);
    float x[8];
    unpack8(raw, x);
    norm_rope_chunk<D>(x, c, is_k ? p.wk : p.wq, p.eps, p.rot, L, p.inv_freq, nullptr);
    const u32x4_t pk = pack8(x);
    float xr[8];
    unpack8(pk, xr);
#pragma unroll
    for (int j = 0; j < 8; ++j) qk[r][c * 8 + j] = xr[j];
    if (is_k) {
      const long slot = (long)b * p.cache_bstride + ((long)L * p.G + g) * D + c * 8;
      *(u32x4_t*)(p.k_cache + slot) = pk;
      *(u32x4_t*)(p.v_cache + slot) = *(const u32x4_t*)(p.v_new + ((long)b * p.G + g) * D + c * 8);
    }
  }
  __syncthreads();
  // the new token's own score, per head
  for (int h = w; h < grp; h += 4) {
    float s = 0.f;
    for (int e = lane; e < D; e += 64) s += qk[h][e] * qk[16][e];
    s = sum_xor<64>(s);
    if (lane == 0) snew[h] = s * p.scale_log2;
  }
  __syncthreads();

  const int ns = (L + kDecodeChunk - 1) / kDecodeChunk;
  const float* ws_o = p.ws;
  const float* ws_ml = p.ws + (long)p.B * p.H * p.nsplit * D;
  // global max and sum per head
  for (int h = w; h < grp; h += 4) {
    const long base = ((long)b * p.H + g * grp + h) * p.nsplit;
    float mx = snew[h];
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, ws_ml[(base + s) * 2]);
    mx = max_xor<64>(mx);
    float sm = 0.f;
    for (int s = lane; s < ns; s += 64) sm += ws_ml[(base + s) * 2 + 1] * __builtin_amdgcn_exp2f(ws_ml[(base + s) * 2] - mx);
    sm = sum_xor<64>(sm) + __builtin_amdgcn_exp2f(snew[h] - mx);
    if (lane == 0) {
      mtot[h] = mx;
      ltot[h] = sm;
    }
  }
  __syncthreads();

  // outputs: thread owns (head, dim) pairs
  constexpr int MAXO = 16 * D / 256;
  float accv[MAXO];
#pragma unroll
  for (int j = 0; j < MAXO; ++j) accv[j] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += SPLITS_PER_PASS) {
    for (int idx = tid; idx < grp * SPLITS_PER_PASS; idx += 256) {
      const int h = idx / SPLITS_PER_PASS, s = idx % SPLITS_PER_PASS;
      const long base = ((long)b * p.H + g * grp + h) * p.nsplit;
      wts[h][s] = (s0 + s < ns) ? __builtin_amdgcn_exp2f(ws_ml[(base + s0 + s) * 2] - mtot[h]) : 0.f;
    }
    __syncthreads();
    const int sn = min(SPLITS_PER_PASS, ns - s0);
#pragma unroll
    for (int j = 0; j < MAXO; ++j) {
      const int idx = tid + 256 * j;
      if (idx < grp * D) {
        const int h = idx / D, e = idx % D;
        const long base = ((long)b * p.H + g * grp + h) * p.nsplit + s0;
        float a = accv[j];
        for (int s = 0; s < sn; ++s) a += ws_o[(base + s) * D + e] * wts[h][s];
        accv[j] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < MAXO; ++j) {
    const int idx = tid + 256 * j;
    if (idx < grp * D) {
      const int h = idx / D, e = idx % D;
      const float vnew = bf16_bits_to_f32(p.v_new[((long)b * p.G + g) * D + e]);
      float y = (accv[j] + vnew * __builtin_amdgcn_exp2f(snew[h] - mtot[h])) / ltot[h];
      if (GATE == 2) y *= sigmoid_f32(bf16_bits_to_f32(p.gate[((long)b * p.H + g * grp + h) * D + e]));
      if (GATE == 1) y *= sigmoid_f32(bf16_bits_to_f32(p.gate[(long)b * p.H + g * grp + h]));
      out[idx] = f32_to_bf16_bits(y);
    }
  }
}

template <int D>
static hipError_t launch_partials_d(const DecodeParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.nsplit, (unsigned)(p.B * p.G));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  const size_t sq = 16 * (D + 8) * 2;
  size_t body = 0;
#define GA_PARTIALS_CASE(GR)                                                                     \
  case GR: {                                                                                     \
    const size_t s1 = (size_t)kDecodeChunk * GR * 4, s2 = (size_t)4 * GR * D * 4;                \
    body = s1 > s2 ? s1 : s2;                                                                    \
    if (sq + body > 65536) {                                                                     \
      hipError_t e = hipFuncSetAttribute((const void*)decode_partials_kernel<D, GR>,             \
                                         hipFuncAttributeMaxDynamicSharedMemorySize,             \
                                         (int)(sq + body));                                      \
      if (e != hipSuccess) return e;                                                             \
    }                                                                                            \
    hipLaunchKernelGGL((decode_partials_kernel<D, GR>), grid, dim3(256), sq + body, s, p);       \
    break;                                                                                       \
  }
  switch (p.grp) {
    GA_PARTIALS_CASE(1)
    GA_PARTIALS_CASE(2)
    GA_PARTIALS_CASE(4)
    GA_PARTIALS_CASE(8)
    GA_PARTIALS_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef GA_PARTIALS_CASE
  return hipGetLastError();
}

hipError_t launch_decode_partials(const DecodeParams& p, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_partials_d<64>(p, s);
    case 128: return launch_partials_d<128>(p, s);
    case 256: return launch_partials_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
static hipError_t launch_merge_d(const DecodeParams& p, int gate_mode, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.G));
  if (grid.x == 0) return hipSuccess;
  switch (gate_mode) {
    case 0: hipLaunchKernelGGL((decode_merge_kernel<D, 0>), grid, dim3(256), 0, s, p); break;
    case 1: hipLaunchKernelGGL((decode_merge_kernel<D, 1>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((decode_merge_kernel<D, 2>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeParams& p, int D, int gate_mode, hipStream_t s) {
  switch (D) {
    case 64: return launch_merge_d<64>(p, gate_mode, s);
    case 128: return launch_merge_d<128>(p, gate_mode, s);
    case 256: return launch_merge_d<256>(p, gate_mode, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ga
