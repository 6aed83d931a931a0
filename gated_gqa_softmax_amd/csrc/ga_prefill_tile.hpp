// Building blocks of the fused prefill kernels (gfx950): the LDS stage ring
// that K-hat and V tiles stream into, the per-wave state of a 32-row query
// group, and one 32-key tile of flash attention on 32x32x16 bf16 MFMA.
//
// Definition: causal softmax(q_hat k_hat^T * scale) V per query head, as in
// "Transformer by Hand · 6. Gated attention" ("The formula"), computed over key
// tiles with a running max and row sum ("Attention, worked all the way
// through", "Why scaling and stable softmax matter").
//
//  * S^T = K Q^T puts one query row per lane (lane l: row l % 32), so the row
//    max needs one permlane32 swap and the probabilities are already in the
//    B-operand layout of O^T += V^T P^T; V^T fragments come from row-major V
//    in LDS through ds_read_b64_tr_b16.
//  * K and V rows are XOR-swizzled in LDS per 16-byte chunk (K: chunk ^
//    (row & 15); V: chunk ^ 4 (row & 3)) so those reads are conflict-free.
//  * Two forms of the softmax. With QK-norm on both sides the scores have a
//    known bound: |q_hat . k_hat| <= |q_hat| |k_hat| and |k_hat| <= sqrt(d)
//    max|w_k| (an RMS-normed row has norm sqrt(d) before its weights; RoPE
//    keeps norms). The bounded tile (attn_tile_b) then subtracts that bound,
//    per query row, inside the QK MFMA (its accumulator starts at -c), so the
//    MFMA result is already the exponent: p = 2^(s - c) <= 1, with no running
//    max, no rescale and no row-max reduction. Subtracting any constant is
//    exact for softmax (it cancels between numerator and denominator); the
//    max is only needed when nothing bounds the scores.
//  * Otherwise (attn_tile) the running max is raised lazily: the output is
//    rescaled only when a tile's max exceeds the reference by more than 2^8,
//    so probabilities stay below 256 (exact in fp32, fine as bf16 operands).
#pragma once

#include "ga_common.hpp"
#include "ga_internal.hpp"

namespace ga {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

template <int D, int NS>
struct TileShape {
  static constexpr int ST = 64;                      // keys per stage
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = ST * ROW_BYTES;  // K (or V) of one stage
  static constexpr int NSTAGE = NS;                 // stage buffers in the ring
  static constexpr int BUF_BYTES = 2 * NSTAGE * TILE_BYTES;
  static constexpr int VBASE = NSTAGE * TILE_BYTES;  // start of the V stages
  static constexpr int LOADS_PER_TILE = TILE_BYTES / 1024;  // 1 KB per wave instruction
  static constexpr int LOADS_PER_WAVE = LOADS_PER_TILE / 8;
  static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;
  static_assert(CPR >= 16, "swizzles need at least 16 chunks per row");
  static_assert(LOADS_PER_WAVE >= 1, "tile too small");
};

__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }

constexpr float kLazyRescale = 8.0f;  // log2 headroom before the output is rescaled

// Q^T operand fragments of a wave's 32 rows (D/16 fragments of 16 bytes).
// For d = 256 they are held as accumulator-shaped blocks (fragment kk is the
// 16-byte piece kk % 4 of raw[kk / 4]): the register allocator then places
// them without the spills it made for sixteen separate pieces at that
// register budget.
template <int D, bool BLOCKS = (D == 256)>
struct QFrags {
  bf16x8_t f[D / 16];
  __device__ __forceinline__ bf16x8_t get(int kk) const { return f[kk]; }
  __device__ __forceinline__ void set(int kk, bf16x8_t x) { f[kk] = x; }
};
template <int D>
struct QFrags<D, true> {
  f32x16_t raw[D / 64];
  __device__ __forceinline__ bf16x8_t get(int kk) const {
    const f32x16_t& b = raw[kk >> 2];
    const int j = (kk & 3) * 4;
    const f32x4_t v = {b[j], b[j + 1], b[j + 2], b[j + 3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
  __device__ __forceinline__ void set(int kk, bf16x8_t x) {
    const f32x4_t v = __builtin_bit_cast(f32x4_t, x);
    const int j = (kk & 3) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[kk >> 2][j + e] = v[e];
  }
};

// Per-wave state of the main loop.
template <int D>
struct WaveState {
  QFrags<D> q;           // Q^T operand fragments of this wave's 32 rows
  f32x16_t o[D / 32];    // O^T accumulators
  f32x16_t cinit;        // bounded tiles, d < 256: -c (the row's score bound) in every element
  float m_run, l_run;    // reference max (log2 domain; bounded tiles at d = 256: -c) and
                         // lane-partial row sum
  int kbase;             // K operand LDS address of step 0 (lane part, phase included);
                         // step kk reads kbase ^ ((kk & 7) << 5), + 256 for kk >= 8
  int vbase;             // V^T operand LDS address of dim block 0 (lane part, phase and
                         // V base included); dim block mb reads vbase ^ ((mb & 3) << 6), + 256 for mb >= 4
  __device__ __forceinline__ bf16x8_t qf(int kk) const { return q.get(kk); }
  __device__ __forceinline__ void set_qf(int kk, bf16x8_t x) { q.set(kk, x); }
};

// Direct-to-LDS loads of one stage (64 keys of K-hat and V) for this wave:
// 1 KB of LDS per instruction, lane l's 16 bytes at slot l. The whole byte
// offset goes in the VGPR operand so the buffer range check sees it.
template <int D, int NS, int BUF>
__device__ __forceinline__ void stage_issue(unsigned char* smem, i32x4_t krs, i32x4_t vrs, int koff, int voff, int w,
                                         int st, int kv_row_bytes) {
  typedef TileShape<D, NS> S;
  const uint32_t kt = lds_addr(smem + BUF * S::TILE_BYTES);
  const uint32_t vt = lds_addr(smem + S::VBASE + BUF * S::TILE_BYTES);
  const int soff = st * S::ST * kv_row_bytes;
  const int jstep = 8 * S::ROWS_PER_LOAD * kv_row_bytes;
  // opaque per call: each load adds its scalar offset instead of keeping one
  // loop-invariant VGPR per load
  asm volatile("" : "+v"(koff), "+v"(voff));
#pragma unroll
  for (int j = 0; j < S::LOADS_PER_WAVE; ++j) {
    const int t = w + 8 * j;
    buffer_load_lds16(krs, kt + t * 1024, koff + soff + j * jstep);
    buffer_load_lds16(vrs, vt + t * 1024, voff + soff + j * jstep);
  }
}

// One 32-key tile for the wave's 32 rows: keys [32 * HALF, 32 * HALF + 32) of
// stage buffer BUF, past the lane part already in ws.kbase / ws.vbase.
// Operand reads run KPF (K) and VPF (V^T) MFMAs ahead of their use, so LDS
// latency overlaps the matrix pipe instead of stalling each MFMA.
template <int D, int NS, int BUF, int HALF>
__device__ __forceinline__ void attn_tile(const unsigned char* smem, WaveState<D>& ws, bool need_mask, int lim,
                                        float sl2) {
  typedef TileShape<D, NS> S;
  constexpr int NK = D / 16;   // QK steps (16 dims each)
  constexpr int NV = D / 16;   // PV MFMAs: 2 key halves x D/32 dim blocks
  constexpr int KPF = (D == 256) ? 3 : 4;  // bounded by the register budget of d = 256
  constexpr int VPF = (D == 256) ? 2 : 3;
  int kb = ws.kbase, vb = ws.vbase;
  // opaque per tile: the per-step addresses stay short-lived temporaries
  asm volatile("" : "+v"(kb), "+v"(vb));
  // each address is its own opaque value, so none is kept alive across the
  // loop (the K steps kk and kk + 8 would otherwise share one register)
  auto kread = [&](int kk) {
    int a = kb ^ ((kk & 7) << 5);
    asm volatile("" : "+v"(a));
    return *(const bf16x8_t*)(smem + a + (BUF * S::TILE_BYTES + HALF * 32 * S::ROW_BYTES + ((kk >> 3) << 8)));
  };
  // V^T fragment rows: keys 16ks + 4(lane/32) + (lane%16)/4 (+8 for slots 4..7)
  auto vread = [&](int t) {
    const int ks = t / (D / 32), mb = t % (D / 32);
    int a = vb ^ ((mb & 3) << 6);
    asm volatile("" : "+v"(a));
    const unsigned char* a1 =
        smem + a + (BUF * S::TILE_BYTES + HALF * 32 * S::ROW_BYTES + ((mb & 4) << 6) + ks * 16 * S::ROW_BYTES);
    const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a1);
    const i16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a1 + 8 * S::ROW_BYTES));
    const u32x4_t av = {__builtin_bit_cast(u32x2_t, v1)[0], __builtin_bit_cast(u32x2_t, v1)[1],
                        __builtin_bit_cast(u32x2_t, v2)[0], __builtin_bit_cast(u32x2_t, v2)[1]};
    return __builtin_bit_cast(bf16x8_t, av);
  };

  bf16x8_t ka[NK];
  f32x16_t s;
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KPF; ++kk) ka[kk] = kread(kk);
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    if (kk + KPF < NK) ka[kk + KPF] = kread(kk + KPF);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], ws.qf(kk), s, 0, 0, 0);
  }
  // keep that order: KPF reads ahead, then one MFMA per read
  __builtin_amdgcn_sched_group_barrier(0x100, KPF, 0);
#pragma unroll
  for (int kk = 0; kk < NK - KPF; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, KPF, 0);
  // the first V^T operands do not depend on the softmax
  bf16x8_t va[NV];
#pragma unroll
  for (int t = 0; t < VPF; ++t) va[t] = vread(t);
  if (need_mask) {
    // s[i] holds key k0 + 8(i/4) + 4hi + (i%4); visible iff 8(i/4) + (i%4) <= lim
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = ((i >> 2) * 8 + (i & 3) <= lim) ? s[i] : -INFINITY;
  }
  float mloc = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, s[i]);
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
    mloc = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  const float mcand = mloc * sl2;
  if (!__all(mcand <= ws.m_run + kLazyRescale)) {
    const float m_new = fmaxf(ws.m_run, mcand);
    const float alpha = __builtin_amdgcn_exp2f(ws.m_run - m_new);
    ws.l_run *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ws.o[mb][i] *= alpha;
    ws.m_run = m_new;
  }
  const float nm = -ws.m_run;
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl2, nm));
    s[i] = pv;
    lsum += pv;
  }
  ws.l_run += lsum;
  bf16x8_t pb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4_t pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(s[ks * 8 + 2 * j], s[ks * 8 + 2 * j + 1]);
    pb[ks] = __builtin_bit_cast(bf16x8_t, pk);
  }
#pragma unroll
  for (int t = 0; t < NV; ++t) {
    if (t + VPF < NV) va[t + VPF] = vread(t + VPF);
    const int ks = t / (D / 32), mb = t % (D / 32);
    ws.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], pb[ks], ws.o[mb], 0, 0, 0);
  }
  // one MFMA, then the two transposed reads of the operand VPF steps ahead
#pragma unroll
  for (int t = 0; t < NV - VPF; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, VPF, 1);
}

// Bounded-score tile: the same 32 keys as attn_tile, for rows whose scores
// (log2 domain, softmax scale folded into q_hat) never exceed their bound c.
// With CINIT the QK chain starts from ws.cinit = -c, so the scores come out
// as s - c; otherwise (d = 256, where the 16 registers of ws.cinit do not fit
// beside two waves per SIMD) ws.m_run = -c is added before the exp.
// p = 2^(s - c) needs one exp each; the row sum is RowSum's.
// The tile is two halves, tile_b_qk (the QK MFMAs) and tile_b_finish
// (softmax and PV), so a wave may run them in different stages.
// Lane-partial row sum of a bounded tile's probabilities. At d < 256 the
// fp32 probabilities are added in four independent chains (plain adds hide
// under the MFMAs; a chain of v_dot2c_f32_bf16 measured 1.4-2.1 % slower
// there). At d = 256, where the register budget is the limit, the bf16 PV
// operands are added two at a time with v_dot2c_f32_bf16 into one chain
// (the four-chain form measured 0.8-2 % slower there).
template <int D, bool FP32 = (D < 256)>
struct RowSum {
  float a[4];
  __device__ __forceinline__ explicit RowSum(float l) : a{l, 0.f, 0.f, 0.f} {}
  // pair k of the tile: probabilities e0, e1 and their bf16 pair w
  __device__ __forceinline__ void add(int k, float e0, float e1, uint32_t w) {
    a[(2 * k) & 3] += e0;
    a[(2 * k + 1) & 3] += e1;
  }
  __device__ __forceinline__ float total() const { return (a[0] + a[1]) + (a[2] + a[3]); }
};
template <int D>
struct RowSum<D, false> {
  float l;
  __device__ __forceinline__ explicit RowSum(float l0) : l(l0) {}
  __device__ __forceinline__ void add(int, float, float, uint32_t w) {
    const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one2, l, false);
  }
  __device__ __forceinline__ float total() const { return l; }
};

template <int D, int NS, int BUF, int HALF>
__device__ __forceinline__ bf16x8_t tile_kread(const unsigned char* smem, int kb, int kk) {
  typedef TileShape<D, NS> S;
  int a = kb ^ ((kk & 7) << 5);
  // d = 256: opaque per read, so that the eight swizzled addresses are not
  // kept live across the loop (no room beside two waves per SIMD); d < 256:
  // they are, which saves an address operation per read
  if (D == 256) asm volatile("" : "+v"(a));
  return *(const bf16x8_t*)(smem + a + (BUF * S::TILE_BYTES + HALF * 32 * S::ROW_BYTES + ((kk >> 3) << 8)));
}

template <int D, int NS, int BUF, int HALF>
__device__ __forceinline__ bf16x8_t tile_vread(const unsigned char* smem, int vb, int t) {
  typedef TileShape<D, NS> S;
  const int ks = t / (D / 32), mb = t % (D / 32);
  int a = vb ^ ((mb & 3) << 6);
  if (D == 256) asm volatile("" : "+v"(a));  // (as in tile_kread)
  const unsigned char* a1 =
      smem + a + (BUF * S::TILE_BYTES + HALF * 32 * S::ROW_BYTES + ((mb & 4) << 6) + ks * 16 * S::ROW_BYTES);
  const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a1);
  const i16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a1 + 8 * S::ROW_BYTES));
  const u32x4_t av = {__builtin_bit_cast(u32x2_t, v1)[0], __builtin_bit_cast(u32x2_t, v1)[1],
                      __builtin_bit_cast(u32x2_t, v2)[0], __builtin_bit_cast(u32x2_t, v2)[1]};
  return __builtin_bit_cast(bf16x8_t, av);
}

template <int D, int NS, int BUF, int HALF, bool CINIT = (D < 256)>
__device__ __forceinline__ f32x16_t tile_b_qk(const unsigned char* smem, const WaveState<D>& ws) {
  constexpr int NK = D / 16;
  constexpr int KPF = (D == 256) ? 3 : 4;
  int kb = ws.kbase;
  if (D == 256) asm volatile("" : "+v"(kb));  // (see tile_kread)
  bf16x8_t ka[NK];
  f32x16_t s;
#pragma unroll
  for (int kk = 0; kk < KPF; ++kk) ka[kk] = tile_kread<D, NS, BUF, HALF>(smem, kb, kk);
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    if (kk + KPF < NK) ka[kk + KPF] = tile_kread<D, NS, BUF, HALF>(smem, kb, kk + KPF);
    if (CINIT)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], ws.qf(kk), kk == 0 ? ws.cinit : s, 0, 0, 0);
    else
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], ws.qf(kk), kk == 0 ? f32x16_t{} : s, 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, KPF, 0);
#pragma unroll
  for (int kk = 0; kk < NK - KPF; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, KPF, 0);
  return s;
}

template <int D, int NS, int BUF, int HALF, bool CINIT = (D < 256)>
__device__ __forceinline__ void tile_b_finish(const unsigned char* smem, WaveState<D>& ws, f32x16_t s,
                                              bool need_mask, int lim) {
  constexpr int NV = D / 16;
  constexpr int VPF = (D == 256) ? 2 : 3;
  int vb = ws.vbase;
  if (D == 256) asm volatile("" : "+v"(vb));
  bf16x8_t va[NV];
#pragma unroll
  for (int t = 0; t < VPF; ++t) va[t] = tile_vread<D, NS, BUF, HALF>(smem, vb, t);
  if (!CINIT) {
    const float nc = ws.m_run;  // -c
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] += nc;
  }
  if (need_mask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = ((i >> 2) * 8 + (i & 3) <= lim) ? s[i] : -INFINITY;
  }
  bf16x8_t pb[2];
  RowSum<D> rs(ws.l_run);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4_t pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e0 = __builtin_amdgcn_exp2f(s[ks * 8 + 2 * j]), e1 = __builtin_amdgcn_exp2f(s[ks * 8 + 2 * j + 1]);
      pk[j] = pack_bf16x2(e0, e1);
      rs.add(j, e0, e1, pk[j]);
    }
    pb[ks] = __builtin_bit_cast(bf16x8_t, pk);
  }
  ws.l_run = rs.total();
#pragma unroll
  for (int t = 0; t < NV; ++t) {
    if (t + VPF < NV) va[t + VPF] = tile_vread<D, NS, BUF, HALF>(smem, vb, t + VPF);
    const int ks = t / (D / 32), mb = t % (D / 32);
    ws.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], pb[ks], ws.o[mb], 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < NV - VPF; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, VPF, 1);
}

// Software-pipelined bounded tiles: the QK MFMAs of the next tile (buffer
// BN, half HN) with the softmax of this tile's scores s between them (the
// exponentials do not wait for the matrix pipe), then this tile's PV (buffer
// B, half H). Returns the next tile's scores. The instruction order is left
// to the compiler.
template <int D, int NS, int B, int H, int BN, int HN, bool CINIT = (D < 256)>
__device__ __forceinline__ f32x16_t tile_b_pipe(const unsigned char* smem, WaveState<D>& ws, f32x16_t s,
                                                bool need_mask, int lim) {
  constexpr int NK = D / 16;
  constexpr int NV = D / 16;
  constexpr int KPF = (D == 256) ? 3 : 2;
  constexpr int VPF = (D == 256) ? 2 : 3;
  constexpr int PPM = (8 + NK - 1) / NK;  // probability pairs per QK MFMA
  if (!CINIT) {
    const float nc = ws.m_run;  // -c
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] += nc;
  }
  if (need_mask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = ((i >> 2) * 8 + (i & 3) <= lim) ? s[i] : -INFINITY;
  }
  int kb = ws.kbase;
  if (D == 256) asm volatile("" : "+v"(kb));  // (see tile_kread)
  bf16x8_t ka[NK];
  f32x16_t sn;
  u32x4_t pk[2];
  RowSum<D> rs(ws.l_run);
#pragma unroll
  for (int kk = 0; kk < KPF; ++kk) ka[kk] = tile_kread<D, NS, BN, HN>(smem, kb, kk);
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    if (kk + KPF < NK) ka[kk + KPF] = tile_kread<D, NS, BN, HN>(smem, kb, kk + KPF);
    if (CINIT)
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], ws.qf(kk), kk == 0 ? ws.cinit : sn, 0, 0, 0);
    else
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], ws.qf(kk), kk == 0 ? f32x16_t{} : sn, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < PPM; ++j) {
      const int k = kk * PPM + j;
      if (k < 8) {
        const float e0 = __builtin_amdgcn_exp2f(s[2 * k]), e1 = __builtin_amdgcn_exp2f(s[2 * k + 1]);
        const uint32_t w = pack_bf16x2(e0, e1);
        pk[k >> 2][k & 3] = w;
        rs.add(k, e0, e1, w);
      }
    }
  }
  ws.l_run = rs.total();
  int vb = ws.vbase;
  if (D == 256) asm volatile("" : "+v"(vb));
  bf16x8_t va[NV];
#pragma unroll
  for (int t = 0; t < VPF; ++t) va[t] = tile_vread<D, NS, B, H>(smem, vb, t);
#pragma unroll
  for (int t = 0; t < NV; ++t) {
    if (t + VPF < NV) va[t + VPF] = tile_vread<D, NS, B, H>(smem, vb, t + VPF);
    const int ks = t / (D / 32), mb = t % (D / 32);
    ws.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], __builtin_bit_cast(bf16x8_t, pk[ks]), ws.o[mb], 0, 0, 0);
  }
  return sn;
}

template <int D, int NS, int BUF, int HALF, bool CINIT = (D < 256)>
__device__ __forceinline__ void attn_tile_b(const unsigned char* smem, WaveState<D>& ws, bool need_mask, int lim) {
  tile_b_finish<D, NS, BUF, HALF, CINIT>(smem, ws, tile_b_qk<D, NS, BUF, HALF, CINIT>(smem, ws), need_mask, lim);
}

// Largest log2-domain score bound a row may have before the bounded tiles'
// probabilities 2^(s - c) could leave the normal fp32 range (the row's
// largest one is at least 2^(-2c)).
constexpr float kMaxScoreBound = 60.0f;

}  // namespace ga
