// K-hat preparation: RMSNorm then partial RoPE of key rows, written once per
// call so that the attention kernels read prepared keys (and so that a KV
// cache holds normed, rotated keys).
//
// QK-Norm before RoPE on keys: "Transformer by Hand · 6. Gated attention",
// section "Four things Qwen3.5 adds to the textbook"; order of operations:
// "Attention, worked all the way through", section "Qwen3's exact order".
#include "ga_common.hpp"
#include "ga_internal.hpp"

namespace ga {

// Generic form (fp32, or bf16 shapes the vector form does not take): one
// 32-lane half-wave per row of d <= 256 elements; lane l holds elements
// l, l+32, ... . The normed row is staged in LDS so that each lane can read
// its RoPE partner (t <-> t + rot/2).
template <typename T>
__global__ __launch_bounds__(256) void prep_keys_kernel(PrepParams p) {
  __shared__ float row_buf[8][256];
  const int hw = threadIdx.x >> 5;
  const int l = threadIdx.x & 31;
  const long nrows = (long)p.B * p.n * p.G;
  const long row = (long)blockIdx.x * 8 + hw;
  bool valid = row < nrows;
  int b = 0, i = 0, g = 0;
  if (valid) {
    g = (int)(row % p.G);
    long t = row / p.G;
    i = (int)(t % p.n);
    b = (int)(t / p.n);
  }
  // chunk against a cache: slot base and real rows of this sequence
  const int base = (valid && p.slot_base) ? p.slot_base[b] : 0;
  const int nb = (valid && p.row_lens) ? p.row_lens[b] : p.n;
  if (base < 0 || base > p.max_base || i >= nb) valid = false;
  const int d = p.d;
  const T* src = (const T*)p.src + (long)b * p.src_bstride + ((long)i * p.G + g) * d;
  float x[8];
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int e = l + 32 * m;
    x[m] = (valid && e < d) ? Elem<T>::load(src, e) : 0.f;
    ss += x[m] * x[m];
  }
  ss = sum_xor<32>(ss);
  const float inv = p.w ? 1.0f / sqrtf(ss / (float)d + p.eps) : 1.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int e = l + 32 * m;
    if (e < d) {
      if (p.w) x[m] = x[m] * inv * p.w[e];
      row_buf[hw][e] = x[m];
    }
  }
  __syncthreads();
  if (!valid) return;
  const int pos = p.positions ? p.positions[(long)b * p.n + i] : base + i;
  const int half = p.rot >> 1;
  const long slot = (long)base + i;
  T* dst = (T*)p.dst + (long)b * p.dst_bstride + (slot * p.G + g) * d;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int e = l + 32 * m;
    if (e >= d) break;
    float y = x[m];
    if (e < p.rot) {
      const bool first = e < half;
      const int t = first ? e : e - half;
      float c, s;
      rope_cos_sin(pos, p.inv_freq[t], &c, &s);
      const float other = row_buf[hw][first ? e + half : e - half];
      y = first ? (x[m] * c - other * s) : (x[m] * c + other * s);
    }
    Elem<T>::store(dst, e, y);
  }
  if (p.vdst) {
    const T* vs = (const T*)p.vsrc + (long)b * p.vsrc_bstride + ((long)i * p.G + g) * d;
    T* vd = (T*)p.vdst + (long)b * p.vdst_bstride + (slot * p.G + g) * d;
    for (int e = l; e < d; e += 32) vd[e] = vs[e];
  }
}

// bf16 rows of d = 64, 128 or 256 with rot % 16 == 0: LPR = d/8 lanes per row,
// 8 elements (16 bytes) per lane, so reads and writes are whole 16-byte row
// pieces. A wave takes kPrepIters groups of 64/LPR rows and issues all its
// reads before using any. One group per wave measured fastest (the kernel is
// latency-bound: more waves in flight beat more rows per wave; 4.2 vs 5.0 us
// for two groups on 4096 tokens x 2 KV heads of d = 256). RoPE partners (t, t + rot/2) sit in lanes c and
// c + rot/16 of the row; only lanes holding rotated chunks evaluate cos/sin.
constexpr int kPrepIters = 1;

template <int D>
__global__ __launch_bounds__(256) void prep_keys_vec_kernel(PrepParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPI = 64 / LPR;
  constexpr int NIT = kPrepIters;
  constexpr int RPW = RPI * NIT;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nrows = p.B * p.n * p.G;  // < 2^31 (checked on the host)
  const int c = lane % LPR;
  const int rsub = lane / LPR;
  const uint16_t* src = (const uint16_t*)p.src;
  const uint16_t* vsrc = (const uint16_t*)p.vsrc;
  uint16_t* dst = (uint16_t*)p.dst;
  uint16_t* vdst = (uint16_t*)p.vdst;
  u32x4_t raw[NIT], vraw[NIT];
  int pos[NIT];
  long drow[NIT], vdrow[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = wave * RPW + it * RPI + rsub;
    bool valid = r < nrows;
    const int rc = valid ? r : 0;  // reads stay in range; invalid rows are not stored
    const int t = rc / p.G;
    const int g = rc - t * p.G;
    const int b = t / p.n;
    const int i = t - b * p.n;
    // chunk against a cache: slot base and real rows of this sequence
    const int base = p.slot_base ? p.slot_base[b] : 0;
    const int nb = p.row_lens ? p.row_lens[b] : p.n;
    if (base < 0 || base > p.max_base || i >= nb) valid = false;
    const long tail = ((long)i * p.G + g) * D + c * 8;
    const long dtail = (((long)base + i) * p.G + g) * D + c * 8;
    raw[it] = *(const u32x4_t*)(src + (long)b * p.src_bstride + tail);
    pos[it] = p.positions ? p.positions[(long)b * p.n + i] : base + i;
    drow[it] = valid ? (long)b * p.dst_bstride + dtail : -1;
    if (vdst) {
      vraw[it] = *(const u32x4_t*)(vsrc + (long)b * p.vsrc_bstride + tail);
      vdrow[it] = (long)b * p.vdst_bstride + dtail;
    }
  }
  float w8[8];
  if (p.w) {
    const f32x4_t a = *(const f32x4_t*)(p.w + c * 8);
    const f32x4_t e = *(const f32x4_t*)(p.w + c * 8 + 4);
    w8[0] = a[0], w8[1] = a[1], w8[2] = a[2], w8[3] = a[3];
    w8[4] = e[0], w8[5] = e[1], w8[6] = e[2], w8[7] = e[3];
  }
  const int half = p.rot >> 1;
  const bool rotated = c * 8 < p.rot;
  const bool first = c * 8 < half;
  const int partner = rotated ? (first ? lane + half / 8 : lane - half / 8) : lane;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float x[8];
    unpack8(raw[it], x);
    if (p.w) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
      ss = group_sum<LPR>(ss);
      const float inv = rsqrtf(ss * (1.0f / D) + p.eps);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= inv * w8[j];
    }
    if (p.rot > 0) {
      float xp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xp[j] = __shfl(x[j], partner, 64);
      if (rotated) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float cs, sn;
          rope_cos_sin(pos[it], p.inv_freq[(first ? c * 8 : c * 8 - half) + j], &cs, &sn);
          x[j] = first ? (x[j] * cs - xp[j] * sn) : (x[j] * cs + xp[j] * sn);
        }
      }
    }
    if (drow[it] >= 0) {
      *(u32x4_t*)(dst + drow[it]) = pack8(x);
      if (vdst) *(u32x4_t*)(vdst + vdrow[it]) = vraw[it];
    }
  }
}

template <int D>
static void launch_vec(const PrepParams& p, hipStream_t s) {
  const long nrows = (long)p.B * p.n * p.G;
  const long rpw = (64 / (D / 8)) * kPrepIters;
  const long waves = (nrows + rpw - 1) / rpw;
  hipLaunchKernelGGL(prep_keys_vec_kernel<D>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, p);
}

hipError_t launch_prep_keys(const PrepParams& p, int is_bf16, hipStream_t s) {
  const long nrows = (long)p.B * p.n * p.G;
  const long blocks = (nrows + 7) / 8;
  if (blocks <= 0) return hipSuccess;
  if (is_bf16 && p.rot % 16 == 0 && (p.d == 64 || p.d == 128 || p.d == 256) && nrows < (1L << 30)) {
    if (p.d == 64) launch_vec<64>(p, s);
    if (p.d == 128) launch_vec<128>(p, s);
    if (p.d == 256) launch_vec<256>(p, s);
    return hipGetLastError();
  }
  if (is_bf16)
    hipLaunchKernelGGL(prep_keys_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(prep_keys_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ga
