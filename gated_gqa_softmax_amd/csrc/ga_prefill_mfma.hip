// Fused flash-style prefill for gfx950, bf16 I/O, fp32 accumulation.
//
// Computes, for every query row (b, i, h), the causal softmax attention of
// RoPE(RMSNorm(q)) against prepared keys K-hat, and the sigmoid output gate:
//   "Transformer by Hand · 6. Gated attention", sections "The formula" and
//   "Four things Qwen3.5 adds to the textbook"; gate placement from
//   "Gated Attention：算完注意力，再决定用多少", section "门放在哪里？";
//   stable softmax from "Attention, worked all the way through", section
//   "Why scaling and stable softmax matter" (here in its online form: a
//   running row max and row sum rescaled as key tiles arrive).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows):
//  * rows are (query head in the GQA group, token) pairs of one KV head, so
//    every K/V tile staged in LDS serves all group heads of TB = 128/group
//    tokens;
//  * each wave owns 32 rows and computes S^T = K Q^T and O^T += V^T P^T with
//    v_mfma_f32_32x32x16_bf16. With S^T, each lane holds scores of one query
//    row, so the row max needs one cross-half swap and the probabilities are
//    already in the B-operand layout of the PV product (no data movement);
//  * V is stored transposed in LDS (key index contiguous) for the A operand;
//  * key tiles above the diagonal are never loaded; only tiles crossing the
//    diagonal (or the sequence end) are masked;
//  * K/V tiles are double buffered: the next tile's global loads are in
//    flight while the current tile is computed;
//  * blocks are dispatched heaviest (last token block) first, and
//    consecutive workgroups alternate KV heads so each XCD's L2 sees few heads.
#include "ga_common.hpp"
#include "ga_gate.hpp"
#include "ga_internal.hpp"

namespace ga {

template <int D, int KN>
struct PrefillShape {
  static constexpr int NW = 4;
  static constexpr int ROWS = 128;
  static constexpr int SK = D + 8;      // K tile row stride (elements)
  static constexpr int SV = KN + 4;     // V^T tile row stride (elements)
  static constexpr int KS_ELEMS = KN * SK;
  static constexpr int VT_ELEMS = D * SV;
  static constexpr int BUF_ELEMS = 2 * (KS_ELEMS + VT_ELEMS);
  static constexpr int QS_ELEMS = ROWS * SK;
  static constexpr int TABLE_ENTRIES = 1024;  // (token, pair) cos/sin entries
  static constexpr int PRO_ELEMS = QS_ELEMS + TABLE_ENTRIES * 4;  // table as float2
  static constexpr int SMEM_ELEMS = BUF_ELEMS > PRO_ELEMS ? BUF_ELEMS : PRO_ELEMS;
  static constexpr int K_ITERS = KN * D / 8 / 256;        // 16-byte K chunks per thread
  static constexpr int V_ITERS = (KN / 2) * (D / 8) / 256;  // key-pair chunks per thread
  static_assert(K_ITERS >= 1 && V_ITERS >= 1, "tile too small for 256 threads");
  static_assert(KN % 32 == 0 && D % 32 == 0, "shape");
};

template <int D, int KN, int GATE>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(const PrefillParams p) {
  typedef PrefillShape<D, KN> S;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::SMEM_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- which (b, g, token block) -------------------------------------------
  const int nBG = p.B * p.G;
  const int u = blockIdx.x;
  const int blk = p.nblk - 1 - u / nBG;
  const int bg = u % nBG;
  const int b = bg / p.G;
  const int g = bg % p.G;
  const int TB = p.TB;
  const int t0 = blk * TB;
  const int n = p.n;
  const int kend = min(n, t0 + TB);
  const int ntiles = (kend + KN - 1) / KN;

  // this lane's query row (as MFMA column l32 of wave w)
  const int my_r = w * 32 + l32;
  const int my_hh = my_r / TB;
  const int my_tt = my_r - my_hh * TB;
  const bool my_valid = (my_hh < p.grp) && (t0 + my_tt < n);
  const int my_tok = my_valid ? t0 + my_tt : 0x3fffffff;
  const int my_h = g * p.grp + my_hh;
  int wave_max_tok = my_valid ? my_tok : -1;
  int wave_min_tok = my_tok;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    wave_max_tok = max(wave_max_tok, __shfl_xor(wave_max_tok, m, 64));
    wave_min_tok = min(wave_min_tok, __shfl_xor(wave_min_tok, m, 64));
  }
  // wave-uniform: keep them in scalar registers so tile skips and masks branch uniformly
  wave_max_tok = __builtin_amdgcn_readfirstlane(wave_max_tok);
  wave_min_tok = __builtin_amdgcn_readfirstlane(wave_min_tok);

  const uint16_t* kbase_ptr = p.khat + (long)b * p.k_bstride + (long)g * D;
  const uint16_t* vbase_ptr = p.v + (long)b * p.v_bstride + (long)g * D;
  const long kv_row = (long)p.G * D;  // elements between consecutive tokens

  // ---- tile loaders ---------------------------------------------------------
  u32x4_t kreg[S::K_ITERS];
  u32x4_t vreg[S::V_ITERS][2];
  auto load_tile = [&](int tile) {
    const int k0 = tile * KN;
#pragma unroll
    for (int it = 0; it < S::K_ITERS; ++it) {
      const int c = tid + 256 * it;
      const int key = c / (D / 8);
      const int dc = c % (D / 8);
      const int kg = k0 + key;
      kreg[it] = (kg < n) ? *(const u32x4_t*)(kbase_ptr + kg * kv_row + dc * 8) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < S::V_ITERS; ++it) {
      const int c = tid + 256 * it;
      const int kp = c % (KN / 2);
      const int dc = c / (KN / 2);
      const int kg = k0 + 2 * kp;
      vreg[it][0] = (kg < n) ? *(const u32x4_t*)(vbase_ptr + kg * kv_row + dc * 8) : u32x4_t{0, 0, 0, 0};
      vreg[it][1] = (kg + 1 < n) ? *(const u32x4_t*)(vbase_ptr + (kg + 1) * kv_row + dc * 8)
                                 : u32x4_t{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Ks = smem + buf * (S::KS_ELEMS + S::VT_ELEMS);
    uint16_t* Vt = Ks + S::KS_ELEMS;
#pragma unroll
    for (int it = 0; it < S::K_ITERS; ++it) {
      const int c = tid + 256 * it;
      const int key = c / (D / 8);
      const int dc = c % (D / 8);
      *(u32x4_t*)(Ks + key * S::SK + dc * 8) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < S::V_ITERS; ++it) {
      const int c = tid + 256 * it;
      const int kp = c % (KN / 2);
      const int dc = c / (KN / 2);
      const u32x4_t a = vreg[it][0];
      const u32x4_t bb = vreg[it][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wa = a[e >> 1];
        const uint32_t wb = bb[e >> 1];
        const uint32_t lo = (e & 1) ? (wa >> 16) : (wa & 0xffffu);
        const uint32_t hi16 = (e & 1) ? (wb & 0xffff0000u) : (wb << 16);
        *(uint32_t*)(Vt + (dc * 8 + e) * S::SV + 2 * kp) = lo | hi16;
      }
    }
  };

  load_tile(0);

  // ---- Q prologue: RMSNorm + RoPE of the 128 rows into LDS (bf16) -----------
  float2* table = (float2*)(smem + S::QS_ELEMS);
  const int half = p.half;
  if (p.use_table) {
    for (int e = tid; e < TB * half; e += 256) {
      const int tt = e / half;
      const int t = e - tt * half;
      const int tok = t0 + tt;
      const int pos = (tok < n) ? (p.positions ? p.positions[(long)b * n + tok] : tok) : 0;
      float c, s;
      rope_cos_sin(pos, p.inv_freq[t], &c, &s);
      table[e] = make_float2(c, s);
    }
    __syncthreads();
  }
  {
    constexpr int LPR = D / 8;       // lanes per row (8 elements each)
    constexpr int RPI = 64 / LPR;    // rows per wave iteration
    const int c = lane % LPR;
    const int rsub = lane / LPR;
    for (int it = 0; it < 32 / RPI; ++it) {
      const int r = w * 32 + it * RPI + rsub;
      const int hh = r / TB;
      const int tt = r - hh * TB;
      const int tok = t0 + tt;
      const bool valid = (hh < p.grp) && (tok < n);
      u32x4_t raw = {0, 0, 0, 0};
      if (valid) {
        const int h = g * p.grp + hh;
        raw = *(const u32x4_t*)(p.q + (((long)b * n + tok) * p.H + h) * p.qs + c * 8);
      }
      float x[8];
      unpack8(raw, x);
      const int pos = valid ? (p.positions ? p.positions[(long)b * n + tok] : tok) : 0;
      norm_rope_chunk<D>(x, c, p.wq ? p.wq + c * 8 : nullptr, p.eps, p.rot, pos, p.inv_freq,
                         p.use_table ? table + tt * half : nullptr);
      *(u32x4_t*)(smem + r * S::SK + c * 8) = pack8(x);
    }
  }
  __syncthreads();
  bf16x8_t qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = *(const bf16x8_t*)(smem + my_r * S::SK + kk * 16 + hi * 8);
  __syncthreads();

  store_tile(0);
  __syncthreads();

  // ---- main loop over key tiles ---------------------------------------------
  f32x16_t o[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;
  float m_run = kNegBig;
  float l_run = 0.f;
  const float sl2 = p.scale_log2;

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) load_tile(tile + 1);
    const int k0 = tile * KN;
    if (k0 <= wave_max_tok) {
      const uint16_t* Ks = smem + buf * (S::KS_ELEMS + S::VT_ELEMS);
      const uint16_t* Vt = Ks + S::KS_ELEMS;
      f32x16_t s[KN / 32];
#pragma unroll
      for (int kb = 0; kb < KN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int kb = 0; kb < KN / 32; ++kb) {
          const bf16x8_t a = *(const bf16x8_t*)(Ks + (kb * 32 + l32) * S::SK + kk * 16 + hi * 8);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
        }
      }
      const bool need_mask = (k0 + KN - 1 > wave_min_tok) || (k0 + KN > n);  // wave-uniform
#pragma unroll
      for (int kb = 0; kb < KN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] *= sl2;
      if (need_mask) {
        const int lim = min(my_tok, n - 1) - (k0 + hi * 4);
#pragma unroll
        for (int kb = 0; kb < KN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            s[kb][i] = (kb * 32 + (i >> 2) * 8 + (i & 3) <= lim) ? s[kb][i] : -INFINITY;
      }
      float mloc = kNegBig;
#pragma unroll
      for (int kb = 0; kb < KN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, s[kb][i]);
      {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
        mloc = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(s[kb][i] - m_new);
          s[kb][i] = pv;
          lsum += pv;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      if (!__all(alpha == 1.0f)) {
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < KN / 32; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4_t pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(s[kb][ks * 8 + 2 * j], s[kb][ks * 8 + 2 * j + 1]);
          const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb) {
            const uint16_t* vr = Vt + (mb * 32 + l32) * S::SV + kb * 32 + ks * 16 + hi * 4;
            const u32x2_t lo = *(const u32x2_t*)vr;
            const u32x2_t hh = *(const u32x2_t*)(vr + 8);
            const u32x4_t av = {lo[0], lo[1], hh[0], hh[1]};
            o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), pb, o[mb], 0, 0, 0);
          }
        }
      }
    }
    if (tile + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, gate, store -------------------------------------
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (!my_valid) return;
  const float inv_l = 1.0f / l_run;
  const long row_off = ((long)b * n + my_tok) * p.H + my_h;  // (b, token, head) index
  if (p.lse && hi == 0) p.lse[row_off] = m_run + __log2f(l_run);
  uint16_t* orow = p.out + row_off * D;
  float hg = 1.0f;
  if (GATE == 1) hg = sigmoid_f32(bf16_bits_to_f32(p.gate[row_off * p.gs]));
  // extended epilogue: the lane pair (l32, 0), (l32, 1) holds the whole row
  float onorm_r = 1.0f;
  long goff = 0;
  if (GATE == kGateExt) {
    if (p.ge.onorm_w) {
      float ss = 0.f;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) ss += (o[mb][j] * inv_l) * (o[mb][j] * inv_l);
      auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
      ss = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      onorm_r = 1.0f / sqrtf(ss * (1.0f / D) + p.ge.onorm_eps);
    }
    goff = ext_gate_offset(p.ge, row_off, p.H);
    if (p.ge.mode == 1) hg = gate_act_f32(bf16_bits_to_f32(p.gate[goff]), p.ge.act);
  }
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int dm = mb * 32 + ig * 8 + hi * 4;
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = o[mb][ig * 4 + j] * inv_l;
      if (GATE == kGateExt) {
        if (p.ge.onorm_w) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = y[j] * onorm_r * p.ge.onorm_w[dm + j];
        }
        if (p.ge.mode == 2) {
          const u32x2_t z = *(const u32x2_t*)(p.gate + goff + dm);
          const float zz[4] = {lo_bf16(z[0]), hi_bf16(z[0]), lo_bf16(z[1]), hi_bf16(z[1])};
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = gate_combine_f32(y[j], gate_act_f32(zz[j], p.ge.act), p.ge.add);
        } else if (p.ge.mode == 1) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = gate_combine_f32(y[j], hg, p.ge.add);
        }
      } else if (GATE == 2) {
        const u32x2_t z = *(const u32x2_t*)(p.gate + row_off * p.gs + dm);
        y[0] *= sigmoid_f32(lo_bf16(z[0]));
        y[1] *= sigmoid_f32(hi_bf16(z[0]));
        y[2] *= sigmoid_f32(lo_bf16(z[1]));
        y[3] *= sigmoid_f32(hi_bf16(z[1]));
      } else if (GATE == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] *= hg;
      }
      const u32x2_t ov = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      *(u32x2_t*)(orow + dm) = ov;
    }
  }
}

template <int D, int KN>
static hipError_t launch_d(const PrefillParams& p, int gate_mode, hipStream_t s) {
  const unsigned grid = (unsigned)(p.B * p.G * p.nblk);
  if (grid == 0) return hipSuccess;
  switch (gate_mode) {
    case 0: hipLaunchKernelGGL((prefill_mfma_kernel<D, KN, 0>), dim3(grid), dim3(256), 0, s, p); break;
    case 1: hipLaunchKernelGGL((prefill_mfma_kernel<D, KN, 1>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((prefill_mfma_kernel<D, KN, 2>), dim3(grid), dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((prefill_mfma_kernel<D, KN, kGateExt>), dim3(grid), dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillParams& p, int D, int gate_mode, hipStream_t s) {
  switch (D) {
    case 64: return launch_d<64, 64>(p, gate_mode, s);
    case 128: return launch_d<128, 64>(p, gate_mode, s);
    case 256: return launch_d<256, 32>(p, gate_mode, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ga
