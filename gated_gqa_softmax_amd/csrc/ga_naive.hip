// Generic gated GQA attention for any head_dim <= 256, fp32 or bf16: one
// wave per query row, keys visited one at a time with an online softmax.
// Serves fp32 inputs and the shapes the fused MFMA kernels do not cover; it
// is latency-bound by design and makes no throughput claim.
//
// Definition: "Transformer by Hand · 6. Gated attention", sections "The
// formula" and "Four things Qwen3.5 adds to the textbook"; the gate as in
// "Gated Attention：算完注意力，再决定用多少", section "门放在哪里？"; decode
// over a cache as in "多头注意力与 GQA", section "标准多头注意力（MHA）".
#include "ga_common.hpp"
#include "ga_internal.hpp"

namespace ga {

// Normalise and rotate one row held as x[m] = row[lane + 64 m], m < 4.
template <typename FreqT>
__device__ void row_norm_rope(float x[4], float* stage, int d, const float* w, float eps, int rot,
                              int pos, const FreqT& inv_freq) {
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) ss += x[m] * x[m];
  ss = sum_xor<64>(ss);
  const float inv = w ? 1.0f / sqrtf(ss / (float)d + eps) : 1.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    if (e < d) {
      if (w) x[m] = x[m] * inv * w[e];
      stage[e] = x[m];
    }
  }
  __syncthreads();
  const int half = rot >> 1;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    if (e < rot) {
      const bool first = e < half;
      const int t = first ? e : e - half;
      float c, s;
      rope_cos_sin(pos, inv_freq[t], &c, &s);
      const float other = stage[first ? e + half : e - half];
      x[m] = first ? (x[m] * c - other * s) : (x[m] * c + other * s);
    }
  }
  __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(64) void naive_kernel(NaiveParams p) {
  __shared__ float stage[256];
  const int lane = threadIdx.x;
  const int H = p.H, G = p.G, d = p.d;
  const int b = blockIdx.y / H;
  const int h = blockIdx.y % H;
  const int grp = H / G;
  const int g = h / grp;
  const int i = blockIdx.x;  // prefill token (decode: 0)
  const float* wq = p.wq;

  int pos, nkeys;
  long qoff, ooff, goff;
  if (p.decode) {
    const int L = p.cache_lens[b];
    qoff = ((long)b * H + h) * p.qs;
    ooff = ((long)b * H + h) * d;
    goff = (long)b * p.ge.gts + (long)h * p.ge.ghs;
    if (L < 0 || L > p.max_len) {
      for (int e = lane; e < d; e += 64) Elem<T>::store((T*)p.out, ooff + e, __builtin_nanf(""));
      return;
    }
    pos = L;
    nkeys = L;  // cached keys; the new token is added after the loop
  } else {
    // chunk against a cache: this row is token base + i of the sequence and
    // sees keys [0, base + i]; padding rows (i >= chunk rows) are not written
    const int base = p.cache_lens ? p.cache_lens[b] : 0;
    const int nb = p.row_lens ? p.row_lens[b] : p.n;
    if (base < 0 || base > p.max_len || i >= nb) return;  // (whole workgroup)
    const long row = ((long)b * p.n + i) * H + h;
    qoff = row * p.qs;
    ooff = row * d;
    goff = ((long)b * p.n + i) * p.ge.gts + (long)h * p.ge.ghs;
    pos = p.positions ? p.positions[(long)b * p.n + i] : base + i;
    nkeys = base + i + 1;
  }

  float qv[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    qv[m] = e < d ? Elem<T>::load((const T*)p.q, qoff + e) : 0.f;
  }
  row_norm_rope(qv, stage, d, wq, p.eps, p.rot, pos, p.inv_freq);

  // decode: prepare the new key (rounded to the storage type, as the cache holds it)
  float kn[4] = {0.f, 0.f, 0.f, 0.f}, vn[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.decode) {
    const long koff = ((long)b * G + g) * d;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      kn[m] = e < d ? Elem<T>::load((const T*)p.k_new, koff + e) : 0.f;
      vn[m] = e < d ? Elem<T>::load((const T*)p.v_new, koff + e) : 0.f;
    }
    row_norm_rope(kn, stage, d, p.wk, p.eps, p.rot, pos, p.inv_freq);
    const long slot = (long)b * p.k_bstride + ((long)pos * G + g) * d;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      if (e < d) {
        T tmp;
        Elem<T>::store(&tmp, 0, kn[m]);
        kn[m] = Elem<T>::load(&tmp, 0);
        if (h % grp == 0) {
          Elem<T>::store((T*)p.k_cache_out, slot + e, kn[m]);
          Elem<T>::store((T*)p.v_cache_out, slot + e, vn[m]);
        }
      }
    }
  }

  const T* K = (const T*)p.khat + (long)b * p.k_bstride + (long)g * d;
  const T* V = (const T*)p.v + (long)b * p.v_bstride + (long)g * d;
  const long stride = (long)G * d;
  float m_run = -INFINITY, l_run = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  const int total = nkeys + (p.decode ? 1 : 0);
  for (int j = 0; j < total; ++j) {
    float kv[4], vv[4];
    const bool is_new = p.decode && j == nkeys;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      if (is_new) {
        kv[m] = kn[m];
        vv[m] = vn[m];
      } else {
        kv[m] = e < d ? Elem<T>::load(K, j * stride + e) : 0.f;
        vv[m] = e < d ? Elem<T>::load(V, j * stride + e) : 0.f;
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) dot += qv[m] * kv[m];
    dot = sum_xor<64>(dot) * p.scale;
    const float m_new = fmaxf(m_run, dot);
    const float alpha = expf(m_run - m_new);
    const float pj = expf(dot - m_new);
    l_run = l_run * alpha + pj;
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = o[m] * alpha + pj * vv[m];
    m_run = m_new;
  }
  // gate variants: act(z) = sigmoid, 0.5 + 0.5 sigmoid, z sigmoid(z) or z;
  // y * act(z) or y + act(z); per-head output RMSNorm first
  const GateEpi& ge = p.ge;
  auto act = [&](float z) {
    const float sg = 1.0f / (1.0f + expf(-z));
    return ge.act == 0 ? sg : ge.act == 1 ? 0.5f + 0.5f * sg : ge.act == 2 ? z * sg : z;
  };
  const float hgate = (p.gate_mode == 1) ? act(Elem<T>::load((const T*)p.gate, goff)) : 1.0f;
  float y[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) y[m] = (lane + 64 * m < d) ? o[m] / l_run : 0.f;
  if (ge.onorm_w) {
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) ss += y[m] * y[m];
    ss = sum_xor<64>(ss);
    const float r = 1.0f / sqrtf(ss / d + ge.onorm_eps);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (lane + 64 * m < d) y[m] = y[m] * r * ge.onorm_w[lane + 64 * m];
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    if (e < d) {
      float v = y[m];
      const float gv = p.gate_mode == 2 ? act(Elem<T>::load((const T*)p.gate, goff + e)) : hgate;
      if (p.gate_mode != 0) v = ge.add ? v + gv : v * gv;
      Elem<T>::store((T*)p.out, ooff + e, v);
    }
  }
}

hipError_t launch_naive(const NaiveParams& p, int is_bf16, hipStream_t s) {
  const dim3 grid(p.decode ? 1u : (unsigned)p.n, (unsigned)(p.B * p.H));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(naive_kernel<uint16_t>, grid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(naive_kernel<float>, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace ga
