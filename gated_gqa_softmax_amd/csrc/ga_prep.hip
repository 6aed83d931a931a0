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

// One 32-lane half-wave per row of d <= 256 elements; lane l holds elements
// l, l+32, ... . The normed row is staged in LDS so that each lane can read
// its RoPE partner (t <-> t + rot/2).
template <typename T>
__global__ __launch_bounds__(256) void prep_keys_kernel(PrepParams p) {
  __shared__ float row_buf[8][256];
  const int hw = threadIdx.x >> 5;
  const int l = threadIdx.x & 31;
  const long nrows = (long)p.B * p.n * p.G;
  const long row = (long)blockIdx.x * 8 + hw;
  const bool valid = row < nrows;
  int b = 0, i = 0, g = 0;
  if (valid) {
    g = (int)(row % p.G);
    long t = row / p.G;
    i = (int)(t % p.n);
    b = (int)(t / p.n);
  }
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
  const int pos = p.positions ? p.positions[(long)b * p.n + i] : i;
  const int half = p.rot >> 1;
  T* dst = (T*)p.dst + (long)b * p.dst_bstride + ((long)i * p.G + g) * d;
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
    T* vd = (T*)p.vdst + (long)b * p.vdst_bstride + ((long)i * p.G + g) * d;
    for (int e = l; e < d; e += 32) vd[e] = vs[e];
  }
}

hipError_t launch_prep_keys(const PrepParams& p, int is_bf16, hipStream_t s) {
  const long nrows = (long)p.B * p.n * p.G;
  const long blocks = (nrows + 7) / 8;
  if (blocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(prep_keys_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(prep_keys_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ga
