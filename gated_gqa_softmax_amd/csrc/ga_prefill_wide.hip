// Fused flash-style prefill for gfx950, wide form for grids with many token
// blocks (batched or long sequences), head_dim 128.
//
// Definition: causal softmax(q_hat k_hat^T * scale) V per query head with
// q_hat = RoPE(RMSNorm(q)) and the sigmoid output gate; sources: "Transformer
// by Hand · 6. Gated attention" ("The formula", "Four things Qwen3.5 adds to
// the textbook"), "Gated Attention：算完注意力，再决定用多少" ("门放在哪里？").
//
// Layout of the work:
//  * A workgroup takes one block of 256 query rows, (head of the GQA group,
//    token) pairs in head-major order, and 8 waves of 32 rows. Every wave reads
//    every K/V stage, so each K/V byte brought into LDS serves 256 rows.
//  * Blocks are dispatched heaviest (latest tokens) first; with many blocks per
//    compute unit the dispatcher then balances the causal triangle.
//  * All waves of a workgroup span about the same key range, so the two waves
//    sharing a SIMD stay equally loaded.
//  * K-hat and V stream through a ring of 4 stages of 64 keys (3 in flight);
//    each wave runs both 32-key tiles of a stage between barriers.
//  * q is read straight into the MFMA operand layout: lane (r, h) holds 16-byte
//    chunks 2kk + h of row r, so the row norm needs the partner lane (r, 1 - h)
//    once and, with rot/2 a multiple of 16, both elements of every RoPE pair
//    sit in the same lane.
//  * The gated output leaves through LDS in row-major order: 16-byte gate
//    reads and output writes.
#include "ga_gate.hpp"
#include "ga_prefill_tile.hpp"

namespace ga {

constexpr int kWideStages = 4;
template <int D>
using WideShape = TileShape<D, kWideStages>;

// Wait until stage st has landed in this wave's part of the ring: `ahead`
// later stages (0 .. kWideStages - 2) may still be in flight.
template <int LPS>
__device__ __forceinline__ void wait_stage(int ahead) {
  static_assert(2 * LPS < 64, "vmcnt range");
  if (ahead >= 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPS) : "memory");
  else if (ahead == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D, int BUF, bool BOUNDED>
__device__ __forceinline__ void wide_step(unsigned char* smem, WaveState<D>& ws, i32x4_t krs, i32x4_t vrs,
                                          int koff, int voff, int w, int st, int nst, int kv_row_bytes,
                                          int wave_min_tok, int wave_max_tok, int my_lim_tok, int n, float sl2,
                                          int hi) {
  typedef WideShape<D> S;
  wait_stage<2 * S::LOADS_PER_WAVE>(min(S::NSTAGE - 2, nst - 1 - st));
  lds_barrier();
  if (st + S::NSTAGE - 1 < nst)
    stage_issue<D, S::NSTAGE, (BUF + S::NSTAGE - 1) % S::NSTAGE>(smem, krs, vrs, koff, voff, w,
                                                                st + S::NSTAGE - 1, kv_row_bytes);
  const int k0 = st * S::ST;
  if (k0 <= wave_max_tok) {
    const bool need_mask = (k0 + 31 > wave_min_tok) || (k0 + 32 > n);
    if (BOUNDED)
      attn_tile_b<D, S::NSTAGE, BUF, 0>(smem, ws, need_mask, my_lim_tok - (k0 + hi * 4));
    else
      attn_tile<D, S::NSTAGE, BUF, 0>(smem, ws, need_mask, my_lim_tok - (k0 + hi * 4), sl2);
  }
  if (k0 + 32 <= wave_max_tok) {
    const bool need_mask = (k0 + 63 > wave_min_tok) || (k0 + 64 > n);
    if (BOUNDED)
      attn_tile_b<D, S::NSTAGE, BUF, 1>(smem, ws, need_mask, my_lim_tok - (k0 + 32 + hi * 4));
    else
      attn_tile<D, S::NSTAGE, BUF, 1>(smem, ws, need_mask, my_lim_tok - (k0 + 32 + hi * 4), sl2);
  }
}

// The main loop, unrolled over the ring.
template <int D, bool BOUNDED>
__device__ __forceinline__ void wide_loop(unsigned char* smem, WaveState<D>& ws, i32x4_t krs, i32x4_t vrs,
                                          int koff, int voff, int w, int nst, int kv_row_bytes, int wave_min_tok,
                                          int wave_max_tok, int my_lim_tok, int n, float sl2, int hi) {
  for (int st0 = 0; st0 < nst; st0 += kWideStages) {
    wide_step<D, 0, BOUNDED>(smem, ws, krs, vrs, koff, voff, w, st0, nst, kv_row_bytes, wave_min_tok, wave_max_tok,
                             my_lim_tok, n, sl2, hi);
    if (st0 + 1 < nst)
      wide_step<D, 1, BOUNDED>(smem, ws, krs, vrs, koff, voff, w, st0 + 1, nst, kv_row_bytes, wave_min_tok,
                               wave_max_tok, my_lim_tok, n, sl2, hi);
    if (st0 + 2 < nst)
      wide_step<D, 2, BOUNDED>(smem, ws, krs, vrs, koff, voff, w, st0 + 2, nst, kv_row_bytes, wave_min_tok,
                               wave_max_tok, my_lim_tok, n, sl2, hi);
    if (st0 + 3 < nst)
      wide_step<D, 3, BOUNDED>(smem, ws, krs, vrs, koff, voff, w, st0 + 3, nst, kv_row_bytes, wave_min_tok,
                               wave_max_tok, my_lim_tok, n, sl2, hi);
  }
}

// Pipelined bounded loop: every tile's softmax and PV run under the QK MFMAs
// of the wave's next tile, also across stages (the second tile of stage st
// finishes under the first QK of stage st + 1). The previous stage's V must
// then survive one more stage: loads run two stages ahead (not three) in the
// four-stage ring. The step has no branches around tiles (tiles past a
// wave's rows are fully masked instead), so the accumulators stay in place;
// before stage 0 the pending tile is an all-masked one over a zeroed V buffer.
template <int D, int BUF>
__device__ __forceinline__ void wide_step_p(unsigned char* smem, WaveState<D>& ws, f32x16_t& cs, bool& cmask,
                                            int& clim, i32x4_t krs, i32x4_t vrs, int koff, int voff, int w, int st,
                                            int nst, int kv_row_bytes, int wave_min_tok, int my_lim_tok, int n,
                                            int hi) {
  typedef WideShape<D> S;
  constexpr int NS = S::NSTAGE;
  constexpr int PB = (BUF + NS - 1) % NS;  // the previous stage's buffer
  wait_stage<2 * S::LOADS_PER_WAVE>(min(1, nst - 1 - st));
  lds_barrier();
  const int k0 = st * S::ST;
  const bool m0 = (k0 + 31 > wave_min_tok) || (k0 + 32 > n), m1 = (k0 + 63 > wave_min_tok) || (k0 + 64 > n);
  const int l0 = my_lim_tok - (k0 + hi * 4), l1 = my_lim_tok - (k0 + 32 + hi * 4);
  const f32x16_t s0 = tile_b_pipe<D, NS, PB, 1, BUF, 0>(smem, ws, cs, cmask, clim);
  // the stage loads go out after the first tile, not in one burst of every
  // wave right after the barrier (same-box A/B: -1.2 to -1.8 %)
  if (st + 2 < nst) stage_issue<D, NS, (BUF + 2) % NS>(smem, krs, vrs, koff, voff, w, st + 2, kv_row_bytes);
  cs = tile_b_pipe<D, NS, BUF, 0, BUF, 1>(smem, ws, s0, m0, l0);
  cmask = m1;
  clim = l1;
}

// Stage st's loads into ring buffer st % kWideStages (a run-time index).
template <int D>
__device__ __forceinline__ void wide_issue_rt(unsigned char* smem, i32x4_t krs, i32x4_t vrs, int koff, int voff, int w,
                                              int st, int kv_row_bytes) {
  switch (st % kWideStages) {
    case 0: stage_issue<D, kWideStages, 0>(smem, krs, vrs, koff, voff, w, st, kv_row_bytes); break;
    case 1: stage_issue<D, kWideStages, 1>(smem, krs, vrs, koff, voff, w, st, kv_row_bytes); break;
    case 2: stage_issue<D, kWideStages, 2>(smem, krs, vrs, koff, voff, w, st, kv_row_bytes); break;
    default: stage_issue<D, kWideStages, 3>(smem, krs, vrs, koff, voff, w, st, kv_row_bytes); break;
  }
}

// The wave computes stages [0, my_nst) (the later ones hold no key its rows
// see), then only takes its part in the loads and barriers of the rest.
template <int D>
__device__ __forceinline__ void wide_loop_p(unsigned char* smem, WaveState<D>& ws, i32x4_t krs, i32x4_t vrs, int koff,
                                            int voff, int w, int nst, int my_nst, int kv_row_bytes, int wave_min_tok,
                                            int my_lim_tok, int n, int hi) {
  f32x16_t cs;
#pragma unroll
  for (int i = 0; i < 16; ++i) cs[i] = -INFINITY;
  bool cmask = false;
  int clim = 0;
  for (int st0 = 0; st0 < my_nst; st0 += kWideStages) {
    wide_step_p<D, 0>(smem, ws, cs, cmask, clim, krs, vrs, koff, voff, w, st0, nst, kv_row_bytes, wave_min_tok,
                      my_lim_tok, n, hi);
    if (st0 + 1 < my_nst)
      wide_step_p<D, 1>(smem, ws, cs, cmask, clim, krs, vrs, koff, voff, w, st0 + 1, nst, kv_row_bytes,
                        wave_min_tok, my_lim_tok, n, hi);
    if (st0 + 2 < my_nst)
      wide_step_p<D, 2>(smem, ws, cs, cmask, clim, krs, vrs, koff, voff, w, st0 + 2, nst, kv_row_bytes,
                        wave_min_tok, my_lim_tok, n, hi);
    if (st0 + 3 < my_nst)
      wide_step_p<D, 3>(smem, ws, cs, cmask, clim, krs, vrs, koff, voff, w, st0 + 3, nst, kv_row_bytes,
                        wave_min_tok, my_lim_tok, n, hi);
  }
  // the last pending tile: its stage's buffer is reloaded two steps later, so
  // not before every wave has passed the next barrier
  typedef WideShape<D> S;
  constexpr int NS = S::NSTAGE;
  switch ((my_nst - 1) % NS) {
    case 0: tile_b_finish<D, NS, 0, 1>(smem, ws, cs, cmask, clim); break;
    case 1: tile_b_finish<D, NS, 1, 1>(smem, ws, cs, cmask, clim); break;
    case 2: tile_b_finish<D, NS, 2, 1>(smem, ws, cs, cmask, clim); break;
    default: tile_b_finish<D, NS, 3, 1>(smem, ws, cs, cmask, clim); break;
  }
  for (int st = my_nst; st < nst; ++st) {
    wait_stage<2 * S::LOADS_PER_WAVE>(min(1, nst - 1 - st));
    lds_barrier();
    if (st + 2 < nst) wide_issue_rt<D>(smem, krs, vrs, koff, voff, w, st + 2, kv_row_bytes);
  }
}

// RoPE of a row held in the MFMA operand layout: x[kk][j] is element
// 16kk + 8hi + j; pair (t, t + 16 HK) for the 16 HK pairs, with the
// frequencies of pairs 16kk + 8hi + j in fr[kk][j].
template <int NK, int HK>
__device__ __forceinline__ void rope_rows(float (&x)[NK][8], const double (&fr)[NK / 2][8], int pos) {
  static_assert(HK <= NK / 2, "rotated pairs");
#pragma unroll
  for (int kk = 0; kk < HK; ++kk)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float c, s;
      rope_cos_sin(pos, fr[kk][j], &c, &s);
      const float a = x[kk][j], e = x[kk + HK][j];
      x[kk][j] = a * c - e * s;
      x[kk + HK][j] = e * c + a * s;
    }
}

template <int D, int GATE>
__global__ __launch_bounds__(512) void prefill_wide_kernel(const PrefillParams p) {
  typedef WideShape<D> S;
  static_assert(256 * D * 4 <= S::BUF_BYTES, "the output staging reuses the stage buffers");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S::BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int nBG = p.B * p.G;
  const int u = blockIdx.x;
  const int blk = p.nblk - 1 - u / nBG;  // heaviest block first
  const int bg = u % nBG;
  const int b = bg / p.G;
  const int g = bg % p.G;
  const int TB = p.TB;
  const int n = p.n;
  const int kend = min(n, blk * TB + TB);
  const int nst = (kend + S::ST - 1) / S::ST;

  // this lane's query row (head-major inside the block). The two waves of a
  // SIMD (w and w + 4) take complementary row slots (wr and 7 - wr's mirror),
  // so the causal diagonal's short rows are spread over the SIMDs.
  const int wr = (w < 4) ? w : 11 - w;
  const int my_r = wr * 32 + l32;
  const int my_hh = my_r / TB;
  const int my_tt = my_r - my_hh * TB;
  const int my_tok0 = blk * TB + my_tt;
  const bool my_valid = (my_hh < p.grp) && (my_tok0 < n);
  const int my_tok = my_valid ? my_tok0 : 0x3fffffff;
  int wave_max_tok = my_valid ? my_tok : -1;
  int wave_min_tok = my_tok;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    wave_max_tok = max(wave_max_tok, __shfl_xor(wave_max_tok, m, 64));
    wave_min_tok = min(wave_min_tok, __shfl_xor(wave_min_tok, m, 64));
  }
  wave_max_tok = __builtin_amdgcn_readfirstlane(wave_max_tok);
  wave_min_tok = __builtin_amdgcn_readfirstlane(wave_min_tok);
  const int my_lim_tok = min(my_tok, n - 1);

  // ---- stage loads: the first NSTAGE - 1 stages go out before anything else
  const int kv_row_bytes = p.G * D * 2;
  const uint32_t valid_bytes = (uint32_t)((n - 1) * kv_row_bytes + D * 2);
  const i32x4_t krs = buffer_desc(p.khat + (long)b * p.k_bstride + (long)g * D, valid_bytes);
  const i32x4_t vrs = buffer_desc(p.v + (long)b * p.v_bstride + (long)g * D, valid_bytes);
  int koff, voff;
  {
    const int row0 = w * S::ROWS_PER_LOAD + lane / S::CPR;
    const int ph = lane % S::CPR;
    koff = row0 * kv_row_bytes + ((ph ^ swz_k(row0)) << 4);
    voff = row0 * kv_row_bytes + ((ph ^ swz_v(row0)) << 4);
  }
  if (nst > 0) stage_issue<D, S::NSTAGE, 0>(smem, krs, vrs, koff, voff, w, 0, kv_row_bytes);
  if (nst > 1) stage_issue<D, S::NSTAGE, 1>(smem, krs, vrs, koff, voff, w, 1, kv_row_bytes);

  // ---- q_hat of this lane's row, straight into the MFMA operand layout -------
  // Lane (l32, hi) holds elements 16kk + 8hi + [0, 8) of row l32 for every kk.
  // Bounded rows fold the softmax scale (log2 domain) into q_hat and start
  // their score accumulators at -c, c = |q_hat| * (bound on |k_hat|).
  // Every global load of the prologue (q, both norm weights, the position,
  // the RoPE frequencies) is issued before any of them is waited for: as a
  // chain of dependent loads they took most of the prologue.
  WaveState<D> ws;
  const float sl2 = p.scale_log2;
  bool bounded;
  {
    constexpr int NK = D / 16;
    const int half = p.half;
    const int hq = my_valid ? g * p.grp + my_hh : g * p.grp;  // rows outside the block read a real row
    const int tq = my_valid ? my_tok0 : 0;
    const uint16_t* qrow = p.q + (((long)b * n + tq) * p.H + hq) * p.qs + hi * 8;
    u32x4_t raw[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) raw[kk] = *(const u32x4_t*)(qrow + kk * 16);
    f32x4_t wv[NK][2];
    if (p.wq) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        wv[kk][0] = *(const f32x4_t*)(p.wq + kk * 16 + hi * 8);
        wv[kk][1] = *(const f32x4_t*)(p.wq + kk * 16 + hi * 8 + 4);
      }
    }
    float wkv[D / 64];
    if (p.wk) {
#pragma unroll
      for (int e = 0; e < D / 64; ++e) wkv[e] = p.wk[lane + 64 * e];
    }
    double fr[NK / 2][8];
#pragma unroll
    for (int kk = 0; kk < NK / 2; ++kk)
      if (kk * 16 < half) {
#pragma unroll
        for (int j = 0; j < 8; ++j) fr[kk][j] = p.inv_freq[kk * 16 + hi * 8 + j];
      }
    const int pos = p.positions ? p.positions[(long)b * n + tq] : tq;

    // score bound: with both norm weights, |s| * log2(e) <= scale * d *
    // max|w_q| * max|w_k| (RMS-normed rows have norm sqrt(d) before their
    // weights, RoPE keeps norms; 2% margin for the bf16 roundings of q_hat and
    // k_hat and the sin/cos error). Workgroup-uniform: it depends on the
    // weights only.
    float mq = 0.f, mk = 0.f;
    if (p.wq) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) mq = fmaxf(mq, fabsf(wv[kk][c2][jj]));
      mq = fmaxf(mq, swap_half(mq));  // the other half of the columns
    }
    if (p.wk) {
#pragma unroll
      for (int e = 0; e < D / 64; ++e) mk = fmaxf(mk, fabsf(wkv[e]));
      mk = max_xor<64>(mk);
    }
    const float kb_norm = mk * sqrtf((float)D) * 1.02f;  // bound on |k_hat|
    bounded = p.wq && p.wk && sl2 * sqrtf((float)D) * mq * kb_norm <= kMaxScoreBound;

    float x[NK][8];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) unpack8(raw[kk], x[kk]);
    // RMSNorm (bounded rows: times the softmax scale); c from the row's norm
    // here, which RoPE keeps
    float c = 0.f;
    if (p.wq) {
      float ss = 0.f;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += x[kk][j] * x[kk][j];
      ss += swap_half(ss);
      const float inv = rsqrtf(ss * (1.0f / D) + p.eps) * (bounded ? sl2 : 1.0f);
      float s2 = 0.f;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[kk][j] *= inv * wv[kk][j >> 2][j & 3];
          s2 += x[kk][j] * x[kk][j];
        }
      if (bounded) c = sqrtf(s2 + swap_half(s2)) * kb_norm;
    }
    // RoPE: pair (t, t + half) with t = 16kk + 8hi + j, kk < half / 16 (the
    // pairing is fixed at compile time for each half / 16)
    switch (half >> 4) {
      case 1: rope_rows<NK, 1>(x, fr, pos); break;
      case 2: rope_rows<NK, 2>(x, fr, pos); break;
      case 3: rope_rows<NK, 3>(x, fr, pos); break;
      case 4: rope_rows<NK, 4>(x, fr, pos); break;
      default: break;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) ws.cinit[i] = -c;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) ws.set_qf(kk, __builtin_bit_cast(bf16x8_t, pack8(x[kk])));
  }
  // the running-max loop keeps three stages in flight, the pipelined one two;
  // the pipelined one starts from an all-masked tile over V buffer NSTAGE - 1,
  // zeroed here (it is first loaded in step 1, after step 0's barrier)
  if (!bounded && nst > 2) stage_issue<D, S::NSTAGE, 2>(smem, krs, vrs, koff, voff, w, 2, kv_row_bytes);
  if (bounded) {
    u32x4_t* zv = (u32x4_t*)(smem + S::VBASE + (S::NSTAGE - 1) * S::TILE_BYTES);
    for (int i = threadIdx.x; i < S::TILE_BYTES / 16; i += 512) zv[i] = u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) ws.o[mb][i] = 0.f;
  ws.m_run = kNegBig;
  ws.l_run = 0.f;
  {
    const int i16 = lane & 15;
    const int g16 = lane >> 4;
    // K operand: row = l32 (+ 32 * HALF), chunk (2kk + hi) ^ (row & 15)
    const int y = lane & 15;
    ws.kbase = l32 * S::ROW_BYTES + ((y >> 1) << 5) + ((hi ^ (y & 1)) << 4);
    // V^T operand: row = 16ks + 4*hi + i16/4 (+8) (+ 32 * HALF), chunk (4mb + c) ^ 4x
    const int x = (i16 >> 2) & 3;
    const int c = (g16 & 1) * 2 + ((i16 & 3) >> 1);
    ws.vbase = S::VBASE + (hi * 4 + (i16 >> 2)) * S::ROW_BYTES + ((4 * x + c) << 4) + (i16 & 1) * 8;
  }

  // ---- main loop ---------------------------------------------------------------
  if (bounded) {
    // stages up to the one holding the wave's last row (at least one)
    const int my_nst = min(nst, max(1, wave_max_tok / S::ST + 1));
    wide_loop_p<D>(smem, ws, krs, vrs, koff, voff, w, nst, my_nst, kv_row_bytes, wave_min_tok, my_lim_tok, n, hi);
  } else {
    wide_loop<D, false>(smem, ws, krs, vrs, koff, voff, w, nst, kv_row_bytes, wave_min_tok, wave_max_tok,
                        my_lim_tok, n, sl2, hi);
  }

  // ---- epilogue: normalise, gate, store ----------------------------------------
  // The wave's 32 rows, RPI rows per instruction and LPR lanes of 8 elements
  // per row. The gate is fetched first so that its latency overlaps the rest.
  constexpr int LPR = D / 8;
  constexpr int RPI = 64 / LPR;
  constexpr int NIT = 32 / RPI;
  const int qc = lane % LPR;
  const int rsub = lane / LPR;
  long erow[NIT];
  u32x4_t graw[NIT];
  uint16_t ghead[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = wr * 32 + it * RPI + rsub;
    const int hh = r / TB;
    const int tt = r - hh * TB;
    const int tok = blk * TB + tt;
    const bool valid = (hh < p.grp) && (tok < n);
    erow[it] = valid ? ((long)b * n + tok) * p.H + g * p.grp + hh : -1;
    const long grow = valid ? erow[it] : ((long)b * n) * p.H + g * p.grp;  // unconditional read
    if (GATE == 2) graw[it] = *(const u32x4_t*)(p.gate + grow * p.gs + qc * 8);
    if (GATE == 1) ghead[it] = p.gate[grow * p.gs];
    if (GATE == kGateExt) {
      graw[it] = u32x4_t{0, 0, 0, 0};
      ghead[it] = 0;
      const long go = ext_gate_offset(p.ge, grow, p.H);
      if (p.ge.mode == 2) graw[it] = *(const u32x4_t*)(p.gate + go + qc * 8);
      else if (p.ge.mode == 1) ghead[it] = p.gate[go];
    }
  }
  float l_run = ws.l_run;
  l_run += swap_half(l_run);
  const float inv_l = 1.0f / l_run;
  lds_barrier();  // every wave is done with the stage buffers
  // the wave's region: 32 rows x D floats, 16-byte chunk q of row r at chunk q ^ (r & 15)
  float* xr = (float*)smem + w * 32 * D;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int q = mb * 8 + ig * 2 + hi;
      f32x4_t y;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) y[jj] = ws.o[mb][ig * 4 + jj] * inv_l;
      *(f32x4_t*)(xr + l32 * D + ((q ^ (l32 & 15)) << 2)) = y;
    }
  // the region is this wave's own: order its LDS writes before its reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (erow[it] < 0) continue;
    const int lr = it * RPI + rsub;
    const f32x4_t y0 = *(const f32x4_t*)(xr + lr * D + (((2 * qc) ^ (lr & 15)) << 2));
    const f32x4_t y1 = *(const f32x4_t*)(xr + lr * D + (((2 * qc + 1) ^ (lr & 15)) << 2));
    float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
    if (GATE == kGateExt) {
      ext_epilogue8<D>(y, p.ge, qc, graw[it], ghead[it]);
    } else if (GATE == 2) {
      float z[8];
      unpack8(graw[it], z);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) y[jj] *= sigmoid_f32(z[jj]);
    } else if (GATE == 1) {
      const float hg = sigmoid_f32(bf16_bits_to_f32(ghead[it]));
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) y[jj] *= hg;
    }
    *(u32x4_t*)(p.out + erow[it] * D + qc * 8) = pack8(y);
  }
}

template <int D>
static hipError_t launch_wide_d(const PrefillParams& p, int gate_mode, hipStream_t s) {
  const long grid = (long)p.B * p.G * p.nblk;
  if (grid <= 0) return hipSuccess;
  switch (gate_mode) {
    case 0: hipLaunchKernelGGL((prefill_wide_kernel<D, 0>), dim3((unsigned)grid), dim3(512), 0, s, p); break;
    case 1: hipLaunchKernelGGL((prefill_wide_kernel<D, 1>), dim3((unsigned)grid), dim3(512), 0, s, p); break;
    case 2: hipLaunchKernelGGL((prefill_wide_kernel<D, 2>), dim3((unsigned)grid), dim3(512), 0, s, p); break;
    default: hipLaunchKernelGGL((prefill_wide_kernel<D, kGateExt>), dim3((unsigned)grid), dim3(512), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_wide(const PrefillParams& p, int D, int gate_mode, hipStream_t s) {
  switch (D) {
    case 128: return launch_wide_d<128>(p, gate_mode, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ga
