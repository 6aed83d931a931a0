// Backward pass of the gated GQA causal attention prefill (bf16 in and out,
// fp32 accumulation), for training the layer of "Transformer by Hand · 6.
// Gated attention" ("How the gate is learned": the gate's gradient
// (y - t) o g(1 - g) x). With dout = dL/dout:
//
//   dy = dout * sigmoid(z),  dz = dout * y * g(1 - g)      (bwd_pre_kernel)
//   P = exp2(s * scale * log2 e - lse),  dP = dy V^T,  dS = P * (dP - rowsum(dy * y))
//   dq_hat = dS k_hat * scale                              (bwd_dq_kernel)
//   dk_hat = sum_heads dS^T q_hat * scale,  dV = sum_heads P^T dy   (bwd_dkv_kernel)
//   dq, dk, dw_q, dw_k through RoPE and RMSNorm           (bwd_norm_rope_kernel)
//
// The attention kernels run on v_mfma_f32_32x32x16_bf16 over copies of
// q-hat, k-hat, v and dy laid out in the MFMA's operand order
// (bwd_blocks_kernel), row-blocked for contractions over dims and
// column-blocked for contractions over tokens, so every operand is one
// coalesced 1 KiB piece. For d = 128 and 256 the staged kernels stream the
// tiles' pieces HBM -> LDS and keep each wave's invariant operands in
// registers; the register-operand kernels (one wave per head, 32 rows and at
// most 128 output dims, pieces read from L2) serve the other shapes. A 32x32
// accumulator holds, in lane l and slot i, row 8(i/4) + 4(l/32) + i%4 and
// column l%32, so a probability tile computed with the key (or query) in the
// column is already the B operand of the product that contracts over the
// other index, provided the A operand holds the same permutation of that
// index: the column-blocked pieces hold tokens 4(l/32) + 0..3 and
// 8 + 4(l/32) + 0..3 of each 16-token step.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "ga_common.hpp"
#include "ga_internal.hpp"

namespace ga {

namespace {

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 4 bytes per lane from byte offset voffset of the buffer straight into LDS
// at lds_base + 4 * lane; waited for like buffer_load_lds16 (ga_common.hpp).
__device__ __forceinline__ void buffer_load_lds4(i32x4_t rsrc, uint32_t lds_base, int voffset) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds_base)
               : "memory");
}

__device__ __forceinline__ bf16x8_t pack_operand(const f32x16_t& x, int half) {
  float f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = x[8 * half + j];
  return __builtin_bit_cast(bf16x8_t, pack8(f));
}

}  // namespace

// ---- gate backward, dy and rowsum(dy * y): one wave per (b, i, h) row -------------
// FROM_OUT: p.y holds the forward's gated output o = y * g instead of y, so
// with g = sigmoid(z): dz = dout * o * (1 - g) and rowsum(dy * y) =
// rowsum(dout * o), with no division by g (which may round to 0).
template <int D, int GATE, bool FROM_OUT = false>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdParams p) {
  constexpr int EPL = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)p.B * p.n * p.H) return;
  const long base = row * D + lane * EPL;
  float y[EPL], go[EPL], z[EPL];
#pragma unroll
  for (int m = 0; m < EPL; ++m) {
    y[m] = bf16_bits_to_f32(p.y[base + m]);
    go[m] = bf16_bits_to_f32(p.dout[base + m]);
    z[m] = GATE == 2 ? bf16_bits_to_f32(p.gate[base + m]) : 0.f;
  }
  float gh = 1.f, dyy = 0.f;
  if (GATE == 1) {
    gh = sigmoid_f32(bf16_bits_to_f32(p.gate[row]));
#pragma unroll
    for (int m = 0; m < EPL; ++m) dyy += go[m] * y[m];
    dyy = sum_xor<64>(dyy);
    if (lane == 0) p.dgate[row] = f32_to_bf16_bits(FROM_OUT ? dyy * (1.f - gh) : dyy * gh * (1.f - gh));
  }
  float ds = 0.f;
#pragma unroll
  for (int m = 0; m < EPL; ++m) {
    const float g = GATE == 2 ? sigmoid_f32(z[m]) : gh;
    if (GATE == 2) p.dgate[base + m] = f32_to_bf16_bits(FROM_OUT ? go[m] * y[m] * (1.f - g) : go[m] * y[m] * g * (1.f - g));
    const uint16_t dyb = f32_to_bf16_bits(GATE == 0 ? go[m] : go[m] * g);
    p.dy_out[base + m] = dyb;
    if (!FROM_OUT || GATE == 0)
      ds += bf16_bits_to_f32(dyb) * y[m];  // the rounded dy the products use
    else if (GATE == 2)
      ds += go[m] * y[m];
  }
  ds = (FROM_OUT && GATE == 1) ? dyy : sum_xor<64>(ds);  // dyy is summed over the row already
  if (lane == 0) p.dsum_out[row] = ds;
}

// ---- MFMA-operand copies ----------------------------------------------------------------
// One thread per 16-byte piece. Row-blocked piece (bh, tb, kk), lane l:
// token tb*32 + l%32, dims kk*16 + 8(l/32) + 0..7. Column-blocked piece
// (bh, db, ts), lane l: dim db*32 + l%32, tokens ts*16 + 4(l/32) + 0..3 and
// ts*16 + 8 + 4(l/32) + 0..3. Tokens >= n read as zero.
__global__ __launch_bounds__(256) void bwd_blocks_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ rb,
                                                         uint16_t* __restrict__ cb, int B, int n, int npad, int HX,
                                                         int D) {
  const long pieces = (long)B * HX * npad * D / 8;  // per layout
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const bool col = idx >= pieces;
  const long k = col ? idx - pieces : idx;
  if (k >= pieces || (col ? cb == nullptr : rb == nullptr)) return;
  const int lane = (int)(k & 63);
  const long piece = k >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  if (!col) {
    const int KK = D / 16;
    const int kk = (int)(piece % KK);
    const long rest = piece / KK;
    const int tb = (int)(rest % (npad / 32));
    const long bh = rest / (npad / 32);
    const int b = (int)(bh / HX), hx = (int)(bh % HX);
    const int t = tb * 32 + l32;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (t < n) v = *(const u32x4_t*)(src + (((long)b * n + t) * HX + hx) * D + kk * 16 + hi * 8);
    *(u32x4_t*)(rb + k * 8) = v;
  } else {
    const int TS = npad / 16;
    const int ts = (int)(piece % TS);
    const long rest = piece / TS;
    const int db = (int)(rest % (D / 32));
    const long bh = rest / (D / 32);
    const int b = (int)(bh / HX), hx = (int)(bh % HX);
    const int e = db * 32 + l32;
    uint16_t h16[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = ts * 16 + (j < 4 ? 4 * hi + j : 8 + 4 * hi + j - 4);
      h16[j] = t < n ? src[(((long)b * n + t) * HX + hx) * D + e] : (uint16_t)0;
    }
    u32x4_t v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (uint32_t)h16[2 * j] | ((uint32_t)h16[2 * j + 1] << 16);
    *(u32x4_t*)(cb + k * 8) = v;
  }
}

__device__ __forceinline__ bf16x8_t piece(const uint16_t* base, long index, int lane) {
  return *(const bf16x8_t*)(base + (index * 64 + lane) * 8);
}

// Two accumulator chains over KK steps: x += piece(kk) bx[kk] and
// y += piece(KK + kk) by[kk], the A operands 1 KiB LDS pieces from base (this
// lane's 16 bytes already added), alternating x and y. The LDS reads run PF
// MFMAs ahead, pinned one read per MFMA, so their latency hides under the
// matrix pipe instead of stalling every MFMA.
// One accumulator chain x += piece(kk) bx[kk] over KK steps, A operands as
// in lds_two_chains.
template <int KK, int PF>
__device__ __forceinline__ void lds_one_chain(const unsigned char* base, const bf16x8_t* bx, f32x16_t& x) {
  bf16x8_t a[KK];
#pragma unroll
  for (int t = 0; t < PF; ++t) a[t] = *(const bf16x8_t*)(base + t * 1024);
#pragma unroll
  for (int t = 0; t < KK; ++t) {
    if (t + PF < KK) a[t + PF] = *(const bf16x8_t*)(base + (t + PF) * 1024);
    x = mfma32(a[t], bx[t], x);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
  for (int t = 0; t < KK - PF; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
}

template <int KK, int PF>
__device__ __forceinline__ void lds_two_chains(const unsigned char* base, const bf16x8_t* bx, const bf16x8_t* by,
                                               f32x16_t& x, f32x16_t& y) {
  constexpr int N = 2 * KK;
  bf16x8_t a[N];
#pragma unroll
  for (int t = 0; t < PF; ++t) a[t] = *(const bf16x8_t*)(base + ((t & 1) * KK + (t >> 1)) * 1024);
#pragma unroll
  for (int t = 0; t < N; ++t) {
    if (t + PF < N) a[t + PF] = *(const bf16x8_t*)(base + (((t + PF) & 1) * KK + ((t + PF) >> 1)) * 1024);
    if (t & 1)
      y = mfma32(a[t], by[t >> 1], y);
    else
      x = mfma32(a[t], bx[t >> 1], x);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
  for (int t = 0; t < N - PF; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
}

// ---- dq-hat: one wave per (b, h, 32 queries, DP output dims) --------------------------
// S^T = K Q^T and dP^T = V dy^T put the query in the accumulator column, so
// dS^T is the B operand of dQ^T += K^T dS^T. A workgroup holds the NPASS dim
// slices of 4 / NPASS consecutive heads and two mirrored query blocks (qb and
// nqb - 1 - qb, so every workgroup has about the same number of key tiles);
// each head's q-hat and dy operands of the current block sit in LDS.
template <int D, int DP>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const BwdParams p) {
  constexpr int NPASS = D / DP, KK = D / 16, DB = D / 32, HPW = 4 / NPASS;
  __shared__ __attribute__((aligned(16))) uint16_t qy_lds[HPW][2][KK * 64 * 8];
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5, w = threadIdx.x >> 6;
  const int nqb = (p.n + 31) / 32, NB = p.npad / 32, TS = p.npad / 16;
  const int hgroups = (p.H + HPW - 1) / HPW;
  const int hgi = (int)(blockIdx.x % ((long)p.B * hgroups));
  const int qpair = (int)(blockIdx.x / ((long)p.B * hgroups));
  const int b = hgi / hgroups, h0 = (hgi % hgroups) * HPW;
  const int hs = w / NPASS, pass = w % NPASS;
  // a wave of a missing head computes on the last head and stores nothing
  const bool active = h0 + hs < p.H;
  const int h = min(h0 + hs, p.H - 1);
  const int bh = b * p.H + h, g = h / p.grp;
  const long bg = (long)b * p.G + g;
  const int d0 = pass * DP;
  for (int half = 0; half < 2; ++half) {
    const int qb = half == 0 ? nqb - 1 - qpair : qpair;  // heavy block first
    if (half == 1 && qb == nqb - 1 - qpair) break;       // (odd middle block: one only)
    __syncthreads();  // the previous block's readers of qy_lds are done
    for (int i = threadIdx.x; i < HPW * KK * 64; i += 256) {
      const int hsl = i / (KK * 64), j = i % (KK * 64);
      const int hq = min(h0 + hsl, p.H - 1);
      const long qp = (((long)b * p.H + hq) * NB + qb) * KK;
      *(u32x4_t*)(qy_lds[hsl][0] + j * 8) = *(const u32x4_t*)(p.q_rb + (qp * 64 + j) * 8);
      *(u32x4_t*)(qy_lds[hsl][1] + j * 8) = *(const u32x4_t*)(p.dy_rb + (qp * 64 + j) * 8);
    }
    __syncthreads();
    const int query = qb * 32 + l32;
    const long qoff = ((long)b * p.n + min(query, p.n - 1)) * p.H + h;
    const float lse = p.lse[qoff], dsum = p.dsum[qoff];
    f32x16_t acc[DP / 32];
#pragma unroll
    for (int mb = 0; mb < DP / 32; ++mb) acc[mb] = f32x16_t{};
    for (int kt = 0; kt <= qb; ++kt) {
      const int k0 = kt * 32;
      const long kpiece = (bg * NB + kt) * KK;
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll 4
      for (int kk = 0; kk < KK; ++kk) {
        s = mfma32(piece(p.k_rb, kpiece + kk, lane), *(const bf16x8_t*)(qy_lds[hs][0] + (kk * 64 + lane) * 8), s);
        dp = mfma32(piece(p.v_rb, kpiece + kk, lane), *(const bf16x8_t*)(qy_lds[hs][1] + (kk * 64 + lane) * 8), dp);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + (i >> 2) * 8 + hi * 4 + (i & 3);
        const bool valid = key <= query && query < p.n;
        const float pv = valid ? __builtin_amdgcn_exp2f(s[i] * p.scale_log2 - lse) : 0.f;
        s[i] = pv * (dp[i] - dsum);  // dS^T
      }
      const bf16x8_t ds0 = pack_operand(s, 0), ds1 = pack_operand(s, 1);
#pragma unroll
      for (int mb = 0; mb < DP / 32; ++mb) {
        const long cpiece = (bg * DB + d0 / 32 + mb) * TS + kt * 2;
        acc[mb] = mfma32(piece(p.k_cb, cpiece, lane), ds0, acc[mb]);
        acc[mb] = mfma32(piece(p.k_cb, cpiece + 1, lane), ds1, acc[mb]);
      }
    }
    if (active && query < p.n) {
      float* dst = p.dqh + (((long)b * p.n + query) * p.H + h) * D + d0;
#pragma unroll
      for (int mb = 0; mb < DP / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[mb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3)] = acc[mb][i] * p.scale;
    }
  }
}

// ---- dq-hat, staged: the key tiles stream through LDS ---------------------------------
// The same products as bwd_dq_kernel. A workgroup holds HPW heads of one KV
// group (NPASS = D / 128 dim slices each, one wave per slice) and a mirrored
// pair of query blocks. The operands of key tile kt that every wave reads
// (row-blocked k-hat and v, KK pieces each, and the column-blocked k-hat of
// all D dims, 2 DB pieces) go HBM -> LDS with direct loads NS - 1 tiles
// ahead, one copy for the four waves; each wave keeps its head's q-hat and dy
// operands of the current block in registers. The pieces are stored in their
// 1 KiB MFMA order, so every LDS operand read is one lane-contiguous b128.
// With two dim slices per head (d = 256) the slices' waves split the tile's
// S and dP: slice 0 holds q-hat and computes S, slice 1 holds dy and computes
// dP, and they swap the tiles through LDS.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_staged_kernel(const BwdParams p) {
  constexpr int DP = 128, NPASS = D / DP, HPW = 4 / NPASS, KK = D / 16, DB = D / 32;
  constexpr int NP = 2 * KK + 2 * DB;  // 1 KiB pieces per stage
  constexpr int NPW = NP / 4;          // direct loads per wave per stage
  constexpr int NS = 3;                // stages in the ring
  static_assert(KK % 4 == 0 && (2 * DB) % 4 == 0 && NPW < 64, "stage split over the four waves");
  __shared__ __attribute__((aligned(16))) unsigned char stg[NS * NP * 1024];
  __shared__ __attribute__((aligned(16))) float xch[NPASS == 2 ? 4 : 1][NPASS == 2 ? 16 * 64 : 1];
  const int lane = threadIdx.x & 63, hi = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nqb = (p.n + 31) / 32, NB = p.npad / 32, TS = p.npad / 16;
  const int hgroups = p.H / HPW;  // the host checks that HPW divides the group size
  const int hgi = (int)(blockIdx.x % ((long)p.B * hgroups));
  const int qpair = (int)(blockIdx.x / ((long)p.B * hgroups));
  const int b = hgi / hgroups, h = (hgi % hgroups) * HPW + w / NPASS;
  const int d0 = (w % NPASS) * DP;
  const long bg = (long)b * p.G + h / p.grp;
  // one KV head's slice of each operand copy: npad * D elements
  const uint32_t slice = (uint32_t)p.npad * D * 2;
  const i32x4_t krs = buffer_desc(p.k_rb + bg * p.npad * D, slice);
  const i32x4_t vrs = buffer_desc(p.v_rb + bg * p.npad * D, slice);
  const i32x4_t crs = buffer_desc(p.k_cb + bg * p.npad * D, slice);
  const uint32_t stg0 = lds_addr(stg);
  // stage piece j: k-hat rows (j < KK), v rows (KK <= j < 2 KK), then the
  // column-blocked k-hat pieces (dim block (j - 2 KK) / 2, 16-key half (j - 2 KK) % 2)
  auto issue = [&](int kt, int buf) {
    const uint32_t base = stg0 + (uint32_t)(buf * NP * 1024);
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int j = w + 4 * i;
      if (i < KK / 4) {
        buffer_load_lds16(krs, base + j * 1024, (kt * KK + j) * 1024 + lane * 16);
      } else if (i < KK / 2) {
        buffer_load_lds16(vrs, base + j * 1024, (kt * KK + j - KK) * 1024 + lane * 16);
      } else {
        const int jj = j - 2 * KK;
        buffer_load_lds16(crs, base + j * 1024, ((jj >> 1) * TS + kt * 2 + (jj & 1)) * 1024 + lane * 16);
      }
    }
  };
  for (int half = 0; half < 2; ++half) {
    const int qb = half == 0 ? nqb - 1 - qpair : qpair;  // heavy block first
    if (half == 1 && qb == nqb - 1 - qpair) break;       // (odd middle block: one only)
    const int T = qb + 1;  // key tiles of this block
    // every wave is done with the previous block's stage buffers
    lds_barrier();
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < T) issue(t, t);
    // the block's own operands land before the tile loop, so no wait the
    // compiler places for them sits behind a later stage's loads
    // q-hat (S) and dy (dP) operands; with the split, slice 0 holds q-hat and slice 1 dy
    constexpr int NOP = NPASS == 2 ? 1 : 2;
    bf16x8_t qo[KK], yo[NOP == 2 ? KK : 1];
    const long qp = (((long)b * p.H + h) * NB + qb) * KK;
    const uint16_t* own = (NPASS == 2 && (w & 1)) ? p.dy_rb : p.q_rb;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qo[kk] = piece(own, qp + kk, lane);
      if constexpr (NOP == 2) yo[kk] = piece(p.dy_rb, qp + kk, lane);
    }
    const int query = qb * 32 + l32;
    const long qoff = ((long)b * p.n + min(query, p.n - 1)) * p.H + h;
    const float lse = p.lse[qoff], dsum = p.dsum[qoff];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      asm volatile("" ::"v"(qo[kk]));
      if constexpr (NOP == 2) asm volatile("" ::"v"(yo[kk]));
    }
    asm volatile("" ::"v"(lse), "v"(dsum));
    f32x16_t acc[DP / 32];
#pragma unroll
    for (int mb = 0; mb < DP / 32; ++mb) acc[mb] = f32x16_t{};
    for (int kt = 0; kt < T; ++kt) {
      // this wave's loads of stage kt are done once at most the later
      // stage's loads are outstanding (loads complete in order)
      if (kt + 1 < T)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NPW) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();  // all of stage kt is in LDS; every wave is past tile kt - 1
      if (kt + NS - 1 < T) issue(kt + NS - 1, (kt + NS - 1) % NS);
      const unsigned char* sb = stg + (kt % NS) * (NP * 1024) + lane * 16;
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      if constexpr (NPASS == 2) {
        // slice 0: S from the k-hat pieces, slice 1: dP from the v pieces; swap
        f32x16_t mine = f32x16_t{};
        lds_one_chain<KK, 4>(sb + (w & 1) * KK * 1024, qo, mine);
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[w][i * 64 + lane] = mine[i];
        lds_barrier();  // both tiles written (the reads of the previous swap ended before this tile's stage barrier)
        f32x16_t other;
#pragma unroll
        for (int i = 0; i < 16; ++i) other[i] = xch[w ^ 1][i * 64 + lane];
        s = (w & 1) ? other : mine;
        dp = (w & 1) ? mine : other;
      } else {
        lds_two_chains<KK, 4>(sb, qo, yo, s, dp);
      }
      // the first column-blocked k-hat operands do not depend on dS
      constexpr int NC = DP / 16, CPF = 4;
      const unsigned char* cb0 = sb + (2 * KK + 2 * (d0 / 32)) * 1024;
      bf16x8_t ca[NC];
#pragma unroll
      for (int t = 0; t < CPF; ++t) ca[t] = *(const bf16x8_t*)(cb0 + t * 1024);
      const int k0 = kt * 32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + (i >> 2) * 8 + hi * 4 + (i & 3);
        const bool valid = key <= query && query < p.n;
        const float pv = __builtin_amdgcn_exp2f(valid ? s[i] * p.scale_log2 - lse : -INFINITY);  // branch-free: exp2(-inf) = 0
        s[i] = pv * (dp[i] - dsum);  // dS^T
      }
      const bf16x8_t ds0 = pack_operand(s, 0), ds1 = pack_operand(s, 1);
      // piece t: dim block d0 / 32 + t / 2, 16-key half t % 2
#pragma unroll
      for (int t = 0; t < NC; ++t) {
        if (t + CPF < NC) ca[t + CPF] = *(const bf16x8_t*)(cb0 + (t + CPF) * 1024);
        acc[t >> 1] = mfma32(ca[t], (t & 1) ? ds1 : ds0, acc[t >> 1]);
      }
    }
    if (query < p.n) {
      float* dst = p.dqh + (((long)b * p.n + query) * p.H + h) * D + d0;
#pragma unroll
      for (int mb = 0; mb < DP / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[mb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3)] = acc[mb][i] * p.scale;
    }
  }
}

// ---- per-head dk-hat and dv: one wave per (b, h, 32 keys, DP output dims) ----------------
// S = Q K^T and dP = dy V^T put the key in the accumulator column, so P and
// dS are the B operands of dV^T += dy^T P and dK^T += Q^T dS. The group's
// heads write separate partials (summed afterwards, in a fixed order). A
// workgroup holds the NPASS dim slices of HPW heads and two mirrored key
// blocks (kb and nkb - 1 - kb, so every workgroup has about the same number
// of query tiles); the current block's k-hat and v operands sit in LDS. With
// two dim slices per head, the slices' waves (w and w ^ 1) share the tile's
// S and dP: one computes S, the other dP, and they swap through LDS
// (double-buffered by tile parity, one barrier per tile). Every wave runs
// every tile so the barriers line up; a wave of a missing head computes on
// the group's last head and stores nothing.
template <int D, int DP>
__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(const BwdParams p) {
  constexpr int NPASS = D / DP, KK = D / 16, DB = D / 32, HPW = 4 / NPASS;
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[2][KK * 64 * 8];
  __shared__ __attribute__((aligned(16))) float xch[NPASS == 2 ? 2 : 1][4][16 * 64];
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5, w = threadIdx.x >> 6;
  const int nkb = (p.n + 31) / 32, NB = p.npad / 32, TS = p.npad / 16;
  const int hgroups = (p.grp + HPW - 1) / HPW;
  const int hg = (int)(blockIdx.x % hgroups);
  const long rest = blockIdx.x / hgroups;
  const int bgi = (int)(rest % ((long)p.B * p.G));
  const int kpair = (int)(rest / ((long)p.B * p.G));
  const int b = bgi / p.G, g = bgi % p.G;
  const long bg = bgi;
  const int pass = w % NPASS, hh = hg * HPW + w / NPASS;
  const bool active = hh < p.grp;
  const int h = g * p.grp + min(hh, p.grp - 1);
  const int bh = b * p.H + h;
  const int d0 = pass * DP;
  for (int half = 0; half < 2; ++half) {
    const int kb = half == 0 ? kpair : nkb - 1 - kpair;  // heavy block first
    if (half == 1 && kb == kpair) break;                 // (odd middle block: one only)
    const long kpiece = (bg * NB + kb) * KK;
    __syncthreads();  // the previous block's readers of kv_lds are done
    for (int i = threadIdx.x; i < KK * 64; i += 256) {
      *(u32x4_t*)(kv_lds[0] + i * 8) = *(const u32x4_t*)(p.k_rb + (kpiece * 64 + i) * 8);
      *(u32x4_t*)(kv_lds[1] + i * 8) = *(const u32x4_t*)(p.v_rb + (kpiece * 64 + i) * 8);
    }
    __syncthreads();
    const int key = kb * 32 + l32;
    f32x16_t dv[DP / 32], dk[DP / 32];
#pragma unroll
    for (int mb = 0; mb < DP / 32; ++mb) dv[mb] = dk[mb] = f32x16_t{};
    for (int qt = kb; qt < nkb; ++qt) {
      const int q0 = qt * 32;
      const long qpiece = ((long)bh * NB + qt) * KK;
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      if constexpr (NPASS == 2) {
        const uint16_t* arow = pass == 0 ? p.q_rb : p.dy_rb;
        const uint16_t* brow = kv_lds[pass];
        f32x16_t mine = f32x16_t{};
#pragma unroll 4
        for (int kk = 0; kk < KK; ++kk)
          mine = mfma32(piece(arow, qpiece + kk, lane), *(const bf16x8_t*)(brow + (kk * 64 + lane) * 8), mine);
        float* xb = xch[qt & 1][0];
#pragma unroll
        for (int i = 0; i < 16; ++i) xb[(w * 16 + i) * 64 + lane] = mine[i];
        __syncthreads();
        f32x16_t other;
#pragma unroll
        for (int i = 0; i < 16; ++i) other[i] = xb[((w ^ 1) * 16 + i) * 64 + lane];
        s = pass == 0 ? mine : other;
        dp = pass == 0 ? other : mine;
      } else {
#pragma unroll 4
        for (int kk = 0; kk < KK; ++kk) {
          s = mfma32(piece(p.q_rb, qpiece + kk, lane), *(const bf16x8_t*)(kv_lds[0] + (kk * 64 + lane) * 8), s);
          dp = mfma32(piece(p.dy_rb, qpiece + kk, lane), *(const bf16x8_t*)(kv_lds[1] + (kk * 64 + lane) * 8), dp);
        }
      }
      // this lane's query row statistics, handed to the lanes whose slots hold that row
      const long ro = ((long)b * p.n + min(q0 + l32, p.n - 1)) * p.H + h;
      const float lse_l = p.lse[ro], dsum_l = p.dsum[ro];
      f32x16_t pm;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = (i >> 2) * 8 + hi * 4 + (i & 3);
        const float lse = __shfl(lse_l, r, 64), dsum = __shfl(dsum_l, r, 64);
        const int query = q0 + r;
        const bool valid = key <= query && query < p.n;
        const float pv = __builtin_amdgcn_exp2f(valid ? s[i] * p.scale_log2 - lse : -INFINITY);  // branch-free: exp2(-inf) = 0
        pm[i] = pv;
        s[i] = pv * (dp[i] - dsum);  // dS
      }
      const bf16x8_t p0 = pack_operand(pm, 0), p1 = pack_operand(pm, 1);
      const bf16x8_t ds0 = pack_operand(s, 0), ds1 = pack_operand(s, 1);
#pragma unroll
      for (int mb = 0; mb < DP / 32; ++mb) {
        const long cpiece = ((long)bh * DB + d0 / 32 + mb) * TS + qt * 2;
        dv[mb] = mfma32(piece(p.dy_cb, cpiece, lane), p0, dv[mb]);
        dv[mb] = mfma32(piece(p.dy_cb, cpiece + 1, lane), p1, dv[mb]);
        dk[mb] = mfma32(piece(p.q_cb, cpiece, lane), ds0, dk[mb]);
        dk[mb] = mfma32(piece(p.q_cb, cpiece + 1, lane), ds1, dk[mb]);
      }
    }
    if (active && key < p.n) {
      const long ko = (((long)b * p.n + key) * p.H + h) * D + d0;
#pragma unroll
      for (int mb = 0; mb < DP / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = mb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
          p.dkp[ko + e] = dk[mb][i] * p.scale;
          p.dvp[ko + e] = dv[mb][i];
        }
    }
  }
}

// ---- per-head dk-hat and dv, staged and pipelined over query tiles ---------------------
// The same products as bwd_dkv_kernel. A workgroup takes one query head and a
// mirrored pair of 64-key super blocks (m and M - 1 - m, two 32-key blocks
// each). Wave w holds key block w & 1 of the super block and a role: role 0
// (w < 2) holds k-hat and computes S, P and dV over all D dims; role 1 holds
// v, computes dP, takes P from its partner (wave w ^ 2) through LDS, and
// computes dS and dK over all D dims. The two MFMA phases of consecutive
// query tiles overlap: the MFMAs that use tile t's P (dV += dy^T P) or dS
// (dK += q-hat^T dS) run interleaved with the same wave's S or dP chain of
// tile t + 1, so the exponentials, the P exchange and the dS arithmetic sit
// between two MFMA phases once per tile. The query tiles' operands go HBM ->
// LDS with direct loads in two rings of two slots, one copy for the four
// waves: the row-blocked q-hat and dy pieces that the chains read, and the
// column-blocked q-hat and dy pieces with the rows' log-sum-exp and rowsum(dy
// y) that the products read. A tile's loads go out one per MFMA pair of the
// previous tile (a burst of them right after the barrier stalls the one wave
// of each SIMD at issue); the columns are waited for at the tile's first
// barrier, the rows before its second.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_pipe_kernel(const BwdParams p) {
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int NR = 2 * KK, NC = 4 * DB;    // 1 KiB pieces per tile: rows, columns
  constexpr int NRW = NR / 4, NCW = NC / 4;  // 16-byte direct loads per wave per tile
  static_assert(KK % 4 == 0 && DB % 2 == 0 && KK == 2 * DB, "pieces split over the four waves");
  __shared__ __attribute__((aligned(16))) unsigned char rows_lds[2][NR * 1024];
  __shared__ __attribute__((aligned(16))) unsigned char cols_lds[2][NC * 1024];
  __shared__ __attribute__((aligned(16))) float stat[2][128];      // [lse of 32 rows x2 | dsum of 32 rows x2]
  __shared__ __attribute__((aligned(16))) float pxch[2][16 * 64];  // P of key block kbw, role 0 -> role 1
  const int lane = threadIdx.x & 63, hi = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int kbw = w & 1, role = w >> 1;
  const int nkb = (p.n + 31) / 32, NB = p.npad / 32, TS = p.npad / 16;
  const int M = (nkb + 1) / 2;  // 64-key super blocks
  const int bh = (int)(blockIdx.x % ((long)p.B * p.H));
  const int spair = (int)(blockIdx.x / ((long)p.B * p.H));
  const int b = bh / p.H, h = bh % p.H;
  const long bg = (long)b * p.G + h / p.grp;
  const uint32_t slice = (uint32_t)p.npad * D * 2;
  const i32x4_t qrs = buffer_desc(p.q_rb + (long)bh * p.npad * D, slice);
  const i32x4_t yrs = buffer_desc(p.dy_rb + (long)bh * p.npad * D, slice);
  const i32x4_t qcs = buffer_desc(p.q_cb + (long)bh * p.npad * D, slice);
  const i32x4_t ycs = buffer_desc(p.dy_cb + (long)bh * p.npad * D, slice);
  const uint32_t nstat = (uint32_t)((long)p.B * p.n * p.H * 4);
  const i32x4_t lrs = buffer_desc(p.lse, nstat), srs = buffer_desc(p.dsum, nstat);
  // row piece j: q-hat rows (j < KK), then dy rows
  auto issue_rows = [&](int qt, int slot) {
    const uint32_t base = lds_addr(rows_lds[slot]);
#pragma unroll
    for (int i = 0; i < NRW; ++i) {
      const int j = w + 4 * i;
      if (i < KK / 4)
        buffer_load_lds16(qrs, base + j * 1024, (qt * KK + j) * 1024 + lane * 16);
      else
        buffer_load_lds16(yrs, base + j * 1024, (qt * KK + j - KK) * 1024 + lane * 16);
    }
  };
  // column piece j: q-hat (j < 2 DB), then dy; dim block jj / 2, 16-query half jj % 2
  auto issue_cols = [&](int qt, int slot) {
    if (w < 2) {  // lanes l and l + 32: row qt * 32 + l (clamped to the last row)
      const int so = ((b * p.n + min(qt * 32 + l32, p.n - 1)) * p.H + h) * 4;
      buffer_load_lds4(w == 0 ? lrs : srs, lds_addr(stat[slot]) + w * 256, so);
    }
    const uint32_t base = lds_addr(cols_lds[slot]);
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      const int j = w + 4 * i;
      const int jj = (i < DB / 2) ? j : j - 2 * DB;
      buffer_load_lds16((i < DB / 2) ? qcs : ycs, base + j * 1024, ((jj >> 1) * TS + qt * 2 + (jj & 1)) * 1024 + lane * 16);
    }
  };
  // single loads of the two rings (load i of this wave), for spreading a
  // tile's loads over the MFMAs: a burst of them right after the barrier
  // stalls the one wave of each SIMD at issue
  auto load_row = [&](int qt, int slot, int i) {
    const int j = w + 4 * i;
    const uint32_t base = lds_addr(rows_lds[slot]);
    if (i < KK / 4)
      buffer_load_lds16(qrs, base + j * 1024, (qt * KK + j) * 1024 + lane * 16);
    else
      buffer_load_lds16(yrs, base + j * 1024, (qt * KK + j - KK) * 1024 + lane * 16);
  };
  auto load_col = [&](int qt, int slot, int i) {
    if (i == 0 && w < 2) {
      const int so = ((b * p.n + min(qt * 32 + l32, p.n - 1)) * p.H + h) * 4;
      buffer_load_lds4(w == 0 ? lrs : srs, lds_addr(stat[slot]) + w * 256, so);
    }
    const int j = w + 4 * i;
    const int jj = (i < DB / 2) ? j : j - 2 * DB;
    buffer_load_lds16((i < DB / 2) ? qcs : ycs, lds_addr(cols_lds[slot]) + j * 1024,
                      ((jj >> 1) * TS + qt * 2 + (jj & 1)) * 1024 + lane * 16);
  };
  for (int half = 0; half < 2; ++half) {
    const int sbk = half == 0 ? spair : M - 1 - spair;  // heavy super block first
    if (half == 1 && sbk == spair) break;               // (odd middle super block: one only)
    const int kb = 2 * sbk + kbw;                       // < NB: npad is a multiple of 64
    const int qt0 = 2 * sbk, T = nkb - qt0;             // query tiles [qt0, nkb), T >= 1
    lds_barrier();  // every wave is done with the previous block's buffers
    issue_rows(qt0, 0);
    issue_cols(qt0, 0);
    if (T > 1) issue_rows(qt0 + 1, 1);
    // role 0: k-hat pieces of the block (S = Q K^T), role 1: v pieces (dP = dy V^T)
    bf16x8_t bo[KK];
    const long kpiece = (bg * NB + kb) * KK;
    const uint16_t* own = role ? p.v_rb : p.k_rb;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) bo[kk] = piece(own, kpiece + kk, lane);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(bo[kk]));  // landed before the loop
    const int key = kb * 32 + l32;
    f32x16_t acc[DB];  // role 0: dV^T, role 1: dK^T, all D dims
#pragma unroll
    for (int mb = 0; mb < DB; ++mb) acc[mb] = f32x16_t{};
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // tile qt0's rows and columns and tile qt0 + 1's rows are in LDS
    f32x16_t x = f32x16_t{};  // role 0: S, role 1: dP of the current tile
    lds_one_chain<KK, 4>(rows_lds[0] + lane * 16 + role * KK * 1024, bo, x);
    // one tile's step: wait, refill both rings, P (role 0) / dS (role 1), then
    // tile t's products, with the chain of tile t + 1 between them when NEXT
    auto step = [&](int t, auto next_tag) {
      constexpr bool NEXT = decltype(next_tag)::value;
      const int q0 = (qt0 + t) * 32;
      // outstanding: tile t's columns and statistics, then tile t + 1's rows
      // (loaded during the previous step's MFMAs); the rows are waited for
      // before the second barrier
      if (NEXT)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NRW) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();  // tile t's columns are in; every wave is past tile t - 1
      const bool more_rows = t + 2 < T;  // (the loads go out during the MFMAs below)
      // rows 8 (i / 4) + 4 hi + i % 4 of slot i
      const float* st = stat[t & 1];
      f32x16_t pm;
      if (role == 0) {
        f32x4_t lse4[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) lse4[ib] = *(const f32x4_t*)(st + ib * 8 + hi * 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int query = q0 + (i >> 2) * 8 + hi * 4 + (i & 3);
          const bool valid = key <= query && query < p.n;
          pm[i] = __builtin_amdgcn_exp2f(valid ? x[i] * p.scale_log2 - lse4[i >> 2][i & 3] : -INFINITY);
          pxch[kbw][i * 64 + lane] = pm[i];
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();  // P written (its reads of tile t - 1 ended before this tile's first barrier); tile t + 1's rows are in
      if (role == 1) {
        f32x4_t dsum4[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) dsum4[ib] = *(const f32x4_t*)(st + 64 + ib * 8 + hi * 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) pm[i] = pxch[kbw][i * 64 + lane] * (x[i] - dsum4[i >> 2][i & 3]);  // dS
      }
      const bf16x8_t o0 = pack_operand(pm, 0), o1 = pack_operand(pm, 1);
      // column piece u: dim block u / 2, 16-query half u % 2 of dy (role 0) or q-hat (role 1)
      const unsigned char* cb = cols_lds[t & 1] + lane * 16 + (role ? 0 : 2 * DB) * 1024;
      constexpr int PF = 2;
      if constexpr (NEXT) {
        // the chain of tile t + 1 (row pieces) interleaved with tile t's products
        const unsigned char* rb = rows_lds[(t + 1) & 1] + lane * 16 + role * KK * 1024;
        bf16x8_t ra[KK], ca[KK];
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          ra[u] = *(const bf16x8_t*)(rb + u * 1024);
          ca[u] = *(const bf16x8_t*)(cb + u * 1024);
        }
#pragma unroll
        for (int u = 0; u < KK; ++u) {
          if (u + PF < KK) {
            ra[u + PF] = *(const bf16x8_t*)(rb + (u + PF) * 1024);
            ca[u + PF] = *(const bf16x8_t*)(cb + (u + PF) * 1024);
          }
          x = mfma32(ra[u], bo[u], u == 0 ? f32x16_t{} : x);
          acc[u >> 1] = mfma32(ca[u], (u & 1) ? o1 : o0, acc[u >> 1]);
          // tile t + 1's columns, then tile t + 2's rows: one load per MFMA pair
          if (u < NCW) load_col(qt0 + t + 1, (t + 1) & 1, u);
          else if (u - NCW < NRW && more_rows) load_row(qt0 + t + 2, t & 1, u - NCW);
        }
        static_assert(NCW + NRW <= KK, "one load per MFMA pair");
        // keep that order: two reads ahead per MFMA pair
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
        for (int u = 0; u < KK - PF; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * PF, 0);
      } else {
        bf16x8_t ca[KK];
#pragma unroll
        for (int u = 0; u < PF; ++u) ca[u] = *(const bf16x8_t*)(cb + u * 1024);
#pragma unroll
        for (int u = 0; u < KK; ++u) {
          if (u + PF < KK) ca[u + PF] = *(const bf16x8_t*)(cb + (u + PF) * 1024);
          acc[u >> 1] = mfma32(ca[u], (u & 1) ? o1 : o0, acc[u >> 1]);
        }
      }
    };
    for (int t = 0; t + 1 < T; ++t) step(t, std::true_type{});
    step(T - 1, std::false_type{});
    if (key < p.n) {
      const long ko_ = (((long)b * p.n + key) * p.H + h) * D;
      float* dst = role ? p.dkp : p.dvp;
      const float sc = role ? p.scale : 1.f;
#pragma unroll
      for (int mb = 0; mb < DB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[ko_ + mb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3)] = acc[mb][i] * sc;
    }
  }
}

// dv[b, j, g] = the group's per-head partials summed in head order, bf16
__global__ __launch_bounds__(256) void bwd_dv_sum_kernel(const float* __restrict__ dvp, uint16_t* __restrict__ dv,
                                                         int B, int n, int H, int G, int D) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)B * n * G * D;
  if (idx >= total) return;
  const int e = (int)(idx % D);
  const long r = idx / D;  // (b*n + j)*G + g
  const long t = r / G;
  const int g = (int)(r % G), grp = H / G;
  const float* src = dvp + (t * H + (long)g * grp) * D + e;
  float acc = 0.f;
  for (int hh = 0; hh < grp; ++hh) acc += src[(long)hh * D];
  dv[idx] = f32_to_bf16_bits(acc);
}

// ---- through RoPE and RMSNorm: each wave takes rows w, w + nwaves, ... ----------------
template <int D>
__global__ __launch_bounds__(256) void bwd_norm_rope_kernel(const BwdNormParams p) {
  constexpr int EPL = D / 64;
  __shared__ float stage[4][D];
  __shared__ float wsum[4][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long rows = (long)p.B * p.n * p.HX;
  const long nwaves = (long)gridDim.x * 4;
  const int half = p.rot / 2;
  float wacc[EPL];
#pragma unroll
  for (int m = 0; m < EPL; ++m) wacc[m] = 0.f;
  for (long row = (long)blockIdx.x * 4 + w; row < rows; row += nwaves) {
    const long t = row / p.HX;  // b * n + i
    const int i = (int)(t % p.n);
    const int pos = p.positions ? p.positions[t] : i;
    float gr[EPL];
    const float* gsrc = p.grad + (t * p.HX * p.gsum + (row - t * p.HX) * p.gsum) * D + lane;
#pragma unroll
    for (int m = 0; m < EPL; ++m) gr[m] = 0.f;
    for (int hh = 0; hh < p.gsum; ++hh)
#pragma unroll
      for (int m = 0; m < EPL; ++m) gr[m] += gsrc[(long)hh * D + 64 * m];
    if (half > 0) {
      // the previous row's reads of stage come before these writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int m = 0; m < EPL; ++m) stage[w][lane + 64 * m] = gr[m];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int m = 0; m < EPL; ++m) {
        const int e = lane + 64 * m;
        if (e < p.rot) {
          const bool first = e < half;
          float c, sn;
          rope_cos_sin(pos, p.inv_freq[first ? e : e - half], &c, &sn);
          const float other = stage[w][first ? e + half : e - half];
          gr[m] = first ? gr[m] * c + other * sn : gr[m] * c - other * sn;
        }
      }
    }
    float dx[EPL];
    if (p.w) {
      float x[EPL], ss = 0.f;
#pragma unroll
      for (int m = 0; m < EPL; ++m) {
        x[m] = bf16_bits_to_f32(p.x[row * D + lane + 64 * m]);
        ss += x[m] * x[m];
      }
      ss = sum_xor<64>(ss);
      const float r = sqrtf(ss / D + p.eps);
      const float inv_r = 1.0f / r;
      float dot = 0.f;
#pragma unroll
      for (int m = 0; m < EPL; ++m) {
        const float xh = x[m] * inv_r;
        dot += gr[m] * p.w[lane + 64 * m] * xh;
        wacc[m] += gr[m] * xh;
      }
      dot = sum_xor<64>(dot) / D;
#pragma unroll
      for (int m = 0; m < EPL; ++m) dx[m] = (gr[m] * p.w[lane + 64 * m] - x[m] * inv_r * dot) * inv_r;
    } else {
#pragma unroll
      for (int m = 0; m < EPL; ++m) dx[m] = gr[m];
    }
#pragma unroll
    for (int m = 0; m < EPL; ++m) p.dx[row * D + lane + 64 * m] = f32_to_bf16_bits(dx[m]);
  }
  if (!p.w || !p.wpart) return;  // (uniform over the workgroup)
#pragma unroll
  for (int m = 0; m < EPL; ++m) wsum[w][lane + 64 * m] = wacc[m];
  __syncthreads();
  for (int e = threadIdx.x; e < D; e += 256)
    p.wpart[(long)blockIdx.x * D + e] = (wsum[0][e] + wsum[1][e]) + (wsum[2][e] + wsum[3][e]);
}

// out[e] = sum over rows r < nrows of part[r][e]
__global__ __launch_bounds__(1024) void bwd_reduce_rows_kernel(const float* part, float* out, int nrows, int d) {
  __shared__ float red[16][64];
  const int e = blockIdx.x * 64 + (threadIdx.x & 63);
  const int w = threadIdx.x >> 6;  // 16 waves, each over rows w, w + 16, ...
  float s = 0.f;
  if (e < d) {
#pragma unroll 8
    for (int r = w; r < nrows; r += 16) s += part[(long)r * d + e];
  }
  red[w][threadIdx.x & 63] = s;
  __syncthreads();
  if (w == 0 && e < d) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += red[k][threadIdx.x];  // fixed order: bit-identical run to run
    out[e] = t;
  }
}

// ---- launchers ----------------------------------------------------------------------------

template <int D>
static hipError_t launch_pre_d(const BwdParams& p, hipStream_t s) {
  const long rows = (long)p.B * p.n * p.H;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (rows == 0) return hipSuccess;
  switch (p.gate_mode + 3 * (p.y_is_out && p.gate_mode != 0)) {
    case 0: hipLaunchKernelGGL((bwd_pre_kernel<D, 0>), dim3(grid), dim3(256), 0, s, p); break;
    case 1: hipLaunchKernelGGL((bwd_pre_kernel<D, 1>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((bwd_pre_kernel<D, 2>), dim3(grid), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((bwd_pre_kernel<D, 1, true>), dim3(grid), dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((bwd_pre_kernel<D, 2, true>), dim3(grid), dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdParams& p, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_pre_d<64>(p, s);
    case 128: return launch_pre_d<128>(p, s);
    case 256: return launch_pre_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_blocks(const uint16_t* src, uint16_t* rb, uint16_t* cb, int B, int n, int npad, int HX, int D,
                             hipStream_t s) {
  const long pieces = (long)B * HX * npad * D / 8;
  if (pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_blocks_kernel, dim3((unsigned)((2 * pieces + 255) / 256)), dim3(256), 0, s, src, rb, cb, B,
                     n, npad, HX, D);
  return hipGetLastError();
}

hipError_t launch_bwd_dv_sum(const float* dvp, uint16_t* dv, int B, int n, int H, int G, int D, hipStream_t s) {
  const long total = (long)B * n * G * D;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dv_sum_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dvp, dv, B, n, H, G,
                     D);
  return hipGetLastError();
}

// The staged kernel serves d = 128 and 256 when its workgroup's heads share
// one KV group and an operand slice fits the buffer loads' 32-bit offsets;
// p.plain selects the register-operand kernel everywhere.
static bool dq_staged_ok(const BwdParams& p, int D) {
  if (D < 128 || p.plain) return false;
  const int hpw = 4 / (D / 128);
  if (p.grp % hpw != 0) return false;
  return (long)p.npad * D * 2 < (1L << 31);
}

template <int D>
static hipError_t launch_dq_d(const BwdParams& p, hipStream_t s) {
  constexpr int DP = D < 128 ? D : 128, HPW = 4 / (D / DP);
  const long pairs = ((p.n + 31) / 32 + 1) / 2;  // mirrored block pairs
  if ((long)p.B * p.H * pairs == 0) return hipSuccess;
  if constexpr (D >= 128) {
    if (dq_staged_ok(p, D)) {
      hipLaunchKernelGGL((bwd_dq_staged_kernel<D>), dim3((unsigned)((long)p.B * (p.H / HPW) * pairs)), dim3(256), 0, s,
                         p);
      return hipGetLastError();
    }
  }
  const long wgs = (long)p.B * ((p.H + HPW - 1) / HPW) * pairs;
  hipLaunchKernelGGL((bwd_dq_kernel<D, DP>), dim3((unsigned)wgs), dim3(256), 0, s, p);
  return hipGetLastError();
}

// p.plain selects the register-operand kernel everywhere.
static bool dkv_staged_ok(const BwdParams& p, int D) {
  if (D < 128 || p.plain) return false;
  return (long)p.npad * D * 2 < (1L << 31) && (long)p.B * p.n * p.H * 4 < (1L << 31);
}

template <int D>
static hipError_t launch_dkv_d(const BwdParams& p, hipStream_t s) {
  constexpr int DP = D < 128 ? D : 128, HPW = 4 / (D / DP);
  if constexpr (D >= 128) {
    if (dkv_staged_ok(p, D)) {
      const long M = ((p.n + 31) / 32 + 1) / 2;  // 64-key super blocks
      const long wgs = (long)p.B * p.H * ((M + 1) / 2);
      if (wgs == 0) return hipSuccess;
      hipLaunchKernelGGL((bwd_dkv_pipe_kernel<D>), dim3((unsigned)wgs), dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  const long wgs = (long)p.B * p.G * (((p.n + 31) / 32 + 1) / 2) * ((p.grp + HPW - 1) / HPW);  // mirrored pairs
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkv_kernel<D, DP>), dim3((unsigned)wgs), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdParams& p, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_dq_d<64>(p, s);
    case 128: return launch_dq_d<128>(p, s);
    case 256: return launch_dq_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dkv(const BwdParams& p, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_dkv_d<64>(p, s);
    case 128: return launch_dkv_d<128>(p, s);
    case 256: return launch_dkv_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_norm_rope(const BwdNormParams& p, int nwg, hipStream_t s) {
  if ((long)p.B * p.n * p.HX == 0) return hipSuccess;
  switch (p.d) {
    case 64: hipLaunchKernelGGL((bwd_norm_rope_kernel<64>), dim3(nwg), dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL((bwd_norm_rope_kernel<128>), dim3(nwg), dim3(256), 0, s, p); break;
    case 256: hipLaunchKernelGGL((bwd_norm_rope_kernel<256>), dim3(nwg), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_reduce_rows(const float* part, float* out, int nrows, int d, hipStream_t s) {
  hipLaunchKernelGGL(bwd_reduce_rows_kernel, dim3((unsigned)((d + 63) / 64)), dim3(1024), 0, s, part, out, nrows,
                     d);
  return hipGetLastError();
}

}  // namespace ga
