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
#include "ga_gate.hpp"
#include "ga_internal.hpp"

namespace ga {

// Work item t of the partials grid: first every whole chunk (sequences in
// order, chunks in order within each), then the last, partial chunk of each
// sequence that has one, so that the grid's last workgroups are short ones and
// the tail of the launch, where the compute units run out of work, is short.
// Lengths outside [0, max_len] count as empty. Wave-uniform; false when t is
// past the last chunk.
template <int C>
__device__ __forceinline__ bool locate_chunk(const int32_t* lens, int B, int max_len, int t, int lane, int& b,
                                             int& split, int& L) {
  int before = 0;  // chunks of the passes and sequences before this 64-sequence window
  for (int pass = 0; pass < 2; ++pass) {
    for (int base = 0; base < B; base += 64) {
      int len = base + lane < B ? lens[base + lane] : 0;
      if (len < 0 || len > max_len) len = 0;
      const int cnt = pass == 0 ? len / C : (len % C != 0 ? 1 : 0);
      int incl = cnt;  // inclusive prefix sum over the window's lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const unsigned long long hit = __ballot(before + incl > t);
      if (hit) {
        const int j = __builtin_ctzll(hit);
        b = base + j;
        L = __shfl(len, j, 64);
        split = pass == 0 ? t - (before + __shfl(incl, j, 64) - __shfl(cnt, j, 64)) : L / C;
        return true;
      }
      before += __shfl(incl, 63, 64);
    }
  }
  return false;
}

template <int D, int GRP>
__global__ __launch_bounds__(256) void decode_partials_kernel(const DecodeParams p) {
  constexpr int C = kDecodeChunk;   // keys per workgroup
  constexpr int SQ = D + 8;
  constexpr int LPR = D / 8;        // lanes per row (8 dims each) in the value mix
  constexpr int KPW = 64 / LPR;     // keys per value-mix step
  constexpr int VSTEPS = 16 / KPW;  // value-mix steps per 16-key group
  __shared__ __attribute__((aligned(16))) uint16_t Qs[16 * SQ];  // q-hat rows (>= GRP are 0)
  __shared__ float Pw[4][16][GRP];                               // per wave: p of the current group
  __shared__ float Aw[4][GRP];                                   // per wave: rescale of the current group
  __shared__ float Xw[4][GRP][D];                                // cross-wave merge: unnormalised o
  __shared__ float Mw[4][GRP], Lw[4][GRP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // consecutive workgroups take the KV heads of one chunk, so the heads'
  // halves of each cache row are read at the same time; the chunks that hold
  // keys come first (whole ones, then the partial ones: locate_chunk), and
  // the grid's surplus (sized for every sequence at max_len) exits at the end
  const int g = blockIdx.x % p.G;
  int b, split, L;
  if (!locate_chunk<C>(p.cache_lens, p.B, p.max_len, (int)(blockIdx.x / p.G), lane, b, split, L)) return;
  const int start = split * C;

  const long row = (long)p.G * D;
  const uint16_t* Kc = p.k_cache + (long)b * p.cache_bstride + (long)g * D;
  const uint16_t* Vc = p.v_cache + (long)b * p.cache_bstride + (long)g * D;
  // The waves take interleaved 16-key groups (wave w: groups w, w + 4, ...),
  // so at any time the workgroup streams one contiguous 64-row window.
  const int kbeg = start + w * 16;
  const int kend = min(start + C, L);
  const int ngroups = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  const float sl2 = p.scale_log2;
  const int dc = lane % LPR, ks = lane / LPR;
  const int l16 = lane & 15, q4 = lane >> 4;

  // ---- every load of the prologue, then the first group's K and V rows, go
  // out before q-hat is computed (as a chain of dependent loads the prologue
  // took about a quarter of a workgroup's life). Lane (r, c) of pass i holds
  // elements [8c, 8c + 8) of q row RP i + r; rows >= GRP are zeros.
  constexpr int RP = 256 / LPR;                  // rows per pass
  constexpr int NQP = (GRP + RP - 1) / RP;       // passes over the group's rows
  const int qr = tid / LPR, qc = tid % LPR;
  u32x4_t qraw[NQP];
#pragma unroll
  for (int i = 0; i < NQP; ++i) {
    qraw[i] = u32x4_t{0, 0, 0, 0};
    if (RP * i + qr < GRP) qraw[i] = *(const u32x4_t*)(p.q + ((long)b * p.H + g * GRP + RP * i + qr) * p.qs + qc * 8);
  }
  f32x4_t qw0 = {0.f, 0.f, 0.f, 0.f}, qw1 = qw0;
  if (p.wq) {
    qw0 = *(const f32x4_t*)(p.wq + qc * 8);
    qw1 = *(const f32x4_t*)(p.wq + qc * 8 + 4);
  }
  const int half = p.rot >> 1;
  const bool first = qc * 8 < half, rotated = qc * 8 < p.rot;
  const int t0 = rotated ? (first ? qc * 8 : qc * 8 - half) : 0;  // pairs t0 .. t0 + 7 (rot % 16 == 0)
  double fr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) fr[j] = p.inv_freq[rotated ? t0 + j : 0];

  float m_lane = kNegBig;  // reference max of head l16 (same in the 4 lanes of that head)
  float l_part = 0.f;      // this lane's share of head l16's row sum
  float acc[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  // K and V rows of the first group; each iteration prefetches the next group
  u32x4_t kr[D / 32];
  u32x4_t vr[VSTEPS];
  // Loads are unconditional: keys past the slice end read the slice's last row
  // (their scores are masked to -inf), so the compiler can track each load.
  const int klast = max(kend - 1, 0);
  {
    const int key = min(kbeg + l16, klast);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) kr[c] = *(const u32x4_t*)(Kc + key * row + c * 32 + q4 * 8);
#pragma unroll
    for (int t = 0; t < VSTEPS; ++t) {
      const int vkey = min(kbeg + ks + KPW * t, klast);
      vr[t] = *(const u32x4_t*)(Vc + vkey * row + dc * 8);
    }
  }

  // q-hat of the group's heads at position L (bf16, the MFMA operand
  // precision): RMSNorm, then RoPE with the partner chunk c +- rot/16
#pragma unroll
  for (int i = 0; i < NQP; ++i) {
    float x[8];
    unpack8(qraw[i], x);
    if (p.wq) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
      ss = group_sum<LPR>(ss);
      const float inv = rsqrtf(ss * (1.0f / D) + p.eps);
      const float w8[8] = {qw0[0], qw0[1], qw0[2], qw0[3], qw1[0], qw1[1], qw1[2], qw1[3]};
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = x[j] * inv * w8[j];
    }
    if (p.rot > 0) {
      const int src = first ? lane + half / 8 : lane - half / 8;
      float xp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xp[j] = __shfl(x[j], rotated ? src : lane, 64);
      if (rotated) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float cs, sn;
          rope_cos_sin(L, fr[j], &cs, &sn);
          x[j] = first ? (x[j] * cs - xp[j] * sn) : (x[j] * cs + xp[j] * sn);
        }
      }
    }
    *(u32x4_t*)(Qs + (RP * i + qr) * SQ + qc * 8) = pack8(x);
  }
  for (int idx = tid + 256 * NQP; idx < 16 * LPR; idx += 256)  // rows past the passes: zeros
    *(u32x4_t*)(Qs + (idx / LPR) * SQ + (idx % LPR) * 8) = u32x4_t{0, 0, 0, 0};
  __syncthreads();
  bf16x8_t qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qf[c] = *(const bf16x8_t*)(Qs + l16 * SQ + c * 32 + q4 * 8);

  for (int gi = 0; gi < ngroups; ++gi) {
    const int k0 = kbeg + gi * 64;
    // scores of this group: S^T[key][head], v_mfma_f32_16x16x32_bf16 over d
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[c]), qf[c], sc, 0, 0, 0);
    // K rows of the next group
    {
      const int key = min(k0 + 64 + l16, klast);
#pragma unroll
      for (int c = 0; c < D / 32; ++c) kr[c] = *(const u32x4_t*)(Kc + key * row + c * 32 + q4 * 8);
    }
    // online softmax of head l16 over the group's keys k0 + 4*q4 + i
    float s[4];
    float gm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = (k0 + q4 * 4 + i < kend) ? sc[i] * sl2 : -INFINITY;
      gm = fmaxf(gm, s[i]);
    }
    gm = fmaxf(gm, __shfl_xor(gm, 16, 64));
    gm = fmaxf(gm, __shfl_xor(gm, 32, 64));
    const float m_new = fmaxf(m_lane, gm);
    const float alpha = __builtin_amdgcn_exp2f(m_lane - m_new);
    m_lane = m_new;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
      ps += s[i];
    }
    l_part = l_part * alpha + ps;
    if (l16 < GRP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Pw[w][q4 * 4 + i][l16] = s[i];
      if (q4 == 0) Aw[w][l16] = alpha;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // value mix: lane owns dims [8dc, 8dc+8) of keys ks + KPW*t
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const float a = Aw[w][h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= a;
    }
    u32x4_t vn[VSTEPS];
#pragma unroll
    for (int t = 0; t < VSTEPS; ++t) {
      const int vkey = min(k0 + 64 + ks + KPW * t, klast);
      vn[t] = *(const u32x4_t*)(Vc + vkey * row + dc * 8);
    }
#pragma unroll
    for (int t = 0; t < VSTEPS; ++t) {
      const int kl = ks + KPW * t;
      float v[8];
      unpack8(vr[t], v);
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        const float pw = Pw[w][kl][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += pw * v[e];
      }
    }
#pragma unroll
    for (int t = 0; t < VSTEPS; ++t) vr[t] = vn[t];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // per-wave totals: row sums over the 4 lanes of each head, o over key slots
  l_part += __shfl_xor(l_part, 16, 64);
  l_part += __shfl_xor(l_part, 32, 64);
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], m, 64);
  if (lane < GRP) {
    Mw[w][lane] = m_lane;
    Lw[w][lane] = l_part;
  }
  if (ks == 0) {
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) Xw[w][h][dc * 8 + e] = acc[h][e];
  }
  __syncthreads();

  // merge the 4 waves and write this chunk's partial result
  float* ws_o = p.ws;
  float* ws_ml = p.ws + (long)p.B * p.H * p.nsplit * D;
  for (int idx = tid; idx < GRP * D; idx += 256) {
    const int h = idx / D, e = idx % D;
    const float M = fmaxf(fmaxf(Mw[0][h], Mw[1][h]), fmaxf(Mw[2][h], Mw[3][h]));
    float o = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) o += Xw[ww][h][e] * __builtin_amdgcn_exp2f(Mw[ww][h] - M);
    ws_o[(((long)b * p.H + g * GRP + h) * p.nsplit + split) * D + e] = o;
    if (e == 0) {
      float l = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) l += Lw[ww][h] * __builtin_amdgcn_exp2f(Mw[ww][h] - M);
      const long mi = ((long)b * p.H + g * GRP + h) * p.nsplit + split;
      ws_ml[mi * 2 + 0] = M;
      ws_ml[mi * 2 + 1] = l;
    }
  }
}

// One workgroup per (sequence, query head): the new token's own key and value,
// the chunk partials, the gate; the group's first head also appends the new
// K-hat and V to the cache. The merge is a handful of small dependent steps,
// so every global load it needs (q and k_new rows, the chunks' (m, l) and
// output rows, v_new, the gate) is issued before the first of them.
template <int D, int GATE>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeParams p) {
  constexpr int LPR = D / 8;      // lanes per q / k row, 8 elements each
  constexpr int PPR = D / 4;      // 16-byte pieces per chunk output row
  constexpr int CPP = 256 / PPR;  // chunks per pass of the workgroup
  constexpr int PF = 16;          // passes held in registers; later chunks are read in a loop
  __shared__ float qk[2][D];      // row 0: q-hat (bf16-rounded); row 1: new k-hat (bf16-rounded)
  __shared__ float red[8];
  __shared__ float wts[256];
  __shared__ __attribute__((aligned(16))) float ored[CPP][D];  // per chunk lane: weighted sums
  __shared__ float sh_snew, sh_M, sh_L;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int grp = p.grp;
  const int g = h / grp;
  const int L = p.cache_lens[b];
  uint16_t* out = p.out + ((long)b * p.H + h) * D;
  if (L < 0 || L > p.max_len) {
    for (int e = tid; e < D; e += 256) out[e] = 0x7fc0;  // NaN
    return;
  }
  const int ns = (L + kDecodeChunk - 1) / kDecodeChunk;
  const long base = ((long)b * p.H + h) * p.nsplit;
  const float* ws_o = p.ws + base * D;
  const float* ws_ml = p.ws + (long)p.B * p.H * p.nsplit * D + base * 2;

  // ---- every load first
  u32x4_t raw = {0, 0, 0, 0};
  if (tid < 2 * LPR) {  // two rows, LPR lanes each (whole lane groups of wave 0)
    const int r = tid / LPR, c = tid % LPR;
    raw = (r == 0) ? *(const u32x4_t*)(p.q + ((long)b * p.H + h) * p.qs + c * 8)
                   : *(const u32x4_t*)(p.k_new + ((long)b * p.G + g) * D + c * 8);
  }
  float m_t = -INFINITY, l_t = 0.f;  // chunk tid's statistics (chunks >= 256 in the loop below)
  if (tid < ns) {
    m_t = ws_ml[tid * 2];
    l_t = ws_ml[tid * 2 + 1];
  }
  const int sub = tid / PPR, e4 = tid % PPR;  // chunk lane, 16-byte piece
  f32x4_t ov[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int sc = sub + CPP * k;
    ov[k] = sc < ns ? *(const f32x4_t*)(ws_o + (long)sc * D + e4 * 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float vnew = 0.f;
  uint16_t graw = 0;
  if (tid < D) {
    vnew = bf16_bits_to_f32(p.v_new[((long)b * p.G + g) * D + tid]);
    if (GATE == 2) graw = p.gate[((long)b * p.H + h) * p.gs + tid];
    if (GATE == 1) graw = p.gate[((long)b * p.H + h) * p.gs];
  }

  // ---- q-hat, new k-hat (appended by the group's first head), own score
  if (tid < 2 * LPR) {
    const int r = tid / LPR, c = tid % LPR;
    float x[8];
    unpack8(raw, x);
    const float* nw = (r == 0) ? p.wq : p.wk;
    norm_rope_chunk<D>(x, c, nw ? nw + c * 8 : nullptr, p.eps, p.rot, L, p.inv_freq, nullptr);
    const u32x4_t pk = pack8(x);
    float xr[8];
    unpack8(pk, xr);
#pragma unroll
    for (int j = 0; j < 8; ++j) qk[r][c * 8 + j] = xr[j];
    if (r == 1 && h % grp == 0) {
      const long slot = (long)b * p.cache_bstride + ((long)L * p.G + g) * D + c * 8;
      *(u32x4_t*)(p.k_cache + slot) = pk;
      *(u32x4_t*)(p.v_cache + slot) = *(const u32x4_t*)(p.v_new + ((long)b * p.G + g) * D + c * 8);
    }
  }
  __syncthreads();
  if (w == 0) {
    float sd = 0.f;
    for (int e = lane; e < D; e += 64) sd += qk[0][e] * qk[1][e];
    sd = sum_xor<64>(sd);
    if (lane == 0) sh_snew = sd * p.scale_log2;
  }
  __syncthreads();
  const float snew = sh_snew;

  // ---- global max over the chunks and the own score
  float mx = fmaxf(snew, m_t);
  for (int sc = tid + 256; sc < ns; sc += 256) mx = fmaxf(mx, ws_ml[sc * 2]);
  mx = max_xor<64>(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  if (tid == 0) sh_M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  const float M = sh_M;

  // ---- row sum, then the weighted sum of the chunk outputs, 256 chunks at a time
  float sm = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += 256) {
    if (s0 > 0) __syncthreads();  // the previous pass's weights are read
    const int sc = s0 + tid;
    if (sc < ns) {
      const float ms = s0 == 0 ? m_t : ws_ml[sc * 2];
      const float ls = s0 == 0 ? l_t : ws_ml[sc * 2 + 1];
      const float wt = __builtin_amdgcn_exp2f(ms - M);
      wts[tid] = wt;
      sm += ls * wt;
    }
    __syncthreads();
    const int sn = min(256, ns - s0);
    if (s0 == 0) {
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        const int c = sub + CPP * k;
        if (c < sn) {
          const float wt = wts[c];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] += ov[k][q] * wt;
        }
      }
    }
    for (int c = sub + CPP * (s0 == 0 ? PF : 0); c < sn; c += CPP) {
      const f32x4_t a = *(const f32x4_t*)(ws_o + (long)(s0 + c) * D + e4 * 4);
      const float wt = wts[c];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += a[q] * wt;
    }
  }
  sm = sum_xor<64>(sm);
  if (lane == 0) red[4 + w] = sm;
  *(f32x4_t*)&ored[sub][e4 * 4] = acc;
  __syncthreads();
  if (tid == 0) sh_L = (red[4] + red[5]) + (red[6] + red[7]) + __builtin_amdgcn_exp2f(snew - M);
  __syncthreads();

  // ---- output
  const int e = tid;
  float y = 0.f;
  if (e < D) {
    float o = 0.f;
#pragma unroll
    for (int c = 0; c < CPP; ++c) o += ored[c][e];
    y = (o + vnew * __builtin_amdgcn_exp2f(snew - M)) / sh_L;
  }
  if (GATE != kGateExt) {
    if (e < D) {
      if (GATE == 2 || GATE == 1) y *= sigmoid_f32(bf16_bits_to_f32(graw));
      out[e] = f32_to_bf16_bits(y);
    }
  } else {
    if (p.ge.onorm_w) {  // per-head RMSNorm of the row over the D threads
      const float ss = sum_xor<64>(y * y);
      if (lane == 0) red[w] = ss;  // red[] was last read before the barrier above
      __syncthreads();
      const float tot = (red[0] + red[1]) + (red[2] + red[3]);
      if (e < D) y = y * (1.0f / sqrtf(tot * (1.0f / D) + p.ge.onorm_eps)) * p.ge.onorm_w[e];
    }
    if (e < D) {
      const long go = (long)b * p.ge.gts + (long)h * p.ge.ghs;
      if (p.ge.mode == 2) y = gate_combine_f32(y, gate_act_f32(bf16_bits_to_f32(p.gate[go + e]), p.ge.act), p.ge.add);
      if (p.ge.mode == 1) y = gate_combine_f32(y, gate_act_f32(bf16_bits_to_f32(p.gate[go]), p.ge.act), p.ge.add);
      out[e] = f32_to_bf16_bits(y);
    }
  }
}

template <int D>
static hipError_t launch_partials_d(const DecodeParams& p, hipStream_t s) {
  const long nwg = (long)p.nsplit * p.B * p.G;
  if (nwg <= 0) return hipSuccess;
  const dim3 grid((unsigned)nwg);
  switch (p.grp) {
    case 1: hipLaunchKernelGGL((decode_partials_kernel<D, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_partials_kernel<D, 2>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_partials_kernel<D, 4>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_partials_kernel<D, 8>), grid, dim3(256), 0, s, p); break;
    case 16: hipLaunchKernelGGL((decode_partials_kernel<D, 16>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
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
  const dim3 grid((unsigned)(p.B * p.H));
  if (grid.x == 0) return hipSuccess;
  switch (gate_mode) {
    case 0: hipLaunchKernelGGL((decode_merge_kernel<D, 0>), grid, dim3(256), 0, s, p); break;
    case 1: hipLaunchKernelGGL((decode_merge_kernel<D, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_merge_kernel<D, 2>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((decode_merge_kernel<D, kGateExt>), grid, dim3(256), 0, s, p); break;
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
