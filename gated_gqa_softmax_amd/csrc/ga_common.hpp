// Device helpers shared by the gfx950 kernels: element conversion, wave
// reductions, RMSNorm/RoPE arithmetic and the sigmoid gate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;  // MFMA operand
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // finite floor for running maxima

// ---- element conversion ----------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even pack of two floats into two bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  typedef float storage;
  static __device__ __forceinline__ float load(const float* p, long i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, long i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {  // bf16 bits
  typedef uint16_t storage;
  static __device__ __forceinline__ float load(const uint16_t* p, long i) { return bf16_bits_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, long i, float x) { p[i] = f32_to_bf16_bits(x); }
};

// ---- arithmetic ------------------------------------------------------------

// Logistic sigmoid in fp32: 1/(1 + 2^(-z*log2 e)) with the hardware
// reciprocal (about 1 ulp). z = 0 gives exactly 0.5; z >= 100 gives exactly
// 1; z <= -100 gives 0.
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// cos/sin of the RoPE angle pos * inv_freq. The angle is formed and reduced
// in fp64, in revolutions (rev = pos * inv_freq / 2pi, reduced to [-1/2, 1/2]),
// so large positions keep full fp32 accuracy; the hardware v_sin_f32 /
// v_cos_f32 then take revolutions directly (measured on gfx950: absolute
// error <= 1.3e-7 on [-1/2, 1/2]).
__device__ __forceinline__ void rope_cos_sin(int pos, double inv_freq, float* c, float* s) {
  const double rev = (double)pos * inv_freq * 0.15915494309189533577;  // 1 / (2 pi)
  const float r = (float)(rev - rint(rev));
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

__device__ __forceinline__ float2 rope_cos_sin_call(int pos, double inv_freq) {
  float c, s;
  rope_cos_sin(pos, inv_freq, &c, &s);
  return make_float2(c, s);
}

// ---- wave reductions (wave64) -----------------------------------------------

template <int WIDTH>
__device__ __forceinline__ float sum_xor(float x) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int WIDTH>
__device__ __forceinline__ float max_xor(float x) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource: 48-bit base, stride 0, num_bytes readable bytes (loads
// at or past num_bytes return zeros), dword 3 = 0x00020000 as for the
// library's other buffer loads. The values are wave-uniform (scalar).
__device__ __forceinline__ i32x4_t buffer_desc(const void* base, uint32_t num_bytes) {
  const unsigned long long a = (unsigned long long)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from byte offset voffset of the buffer straight into LDS
// at lds_base + 16 * lane (lds_base wave-uniform). Written as inline asm so
// the compiler does not track it: a tracked LDS write of unknown extent makes
// the compiler wait for it before every later LDS access, which would
// serialise the loads with the compute they should overlap. The caller waits
// with s_waitcnt vmcnt and a barrier before the data is read.
__device__ __forceinline__ void buffer_load_lds16(i32x4_t rsrc, uint32_t lds_base, int voffset) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds_base)
               : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Sum over the 4 lanes of a quad (lanes 4k..4k+3), all lanes active: two
// DPP quad permutations (xor 1, xor 2), no LDS traffic.
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  return x;
}

// Sum over aligned groups of WIDTH lanes (4, 8, 16 or 32), every lane of a
// group receiving the total, all lanes active: DPP quad permutations, then
// half-row and row mirrors (VALU only), then one xor-16 shuffle for 32.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(WIDTH == 4 || WIDTH == 8 || WIDTH == 16 || WIDTH == 32, "group width");
  x = quad_sum(x);
  if (WIDTH >= 8) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  if (WIDTH >= 16) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
  if (WIDTH >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// Workgroup barrier for LDS traffic only: the wave's LDS operations complete
// before it, while its global loads (including loads into LDS, which the
// caller waits for with an explicit vmcnt) stay in flight. __syncthreads()
// would also wait for every outstanding global load.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Value of lane (l ^ 32) via v_permlane32_swap (gfx950).
__device__ __forceinline__ float swap_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0]: lanes 0-31 keep x, lanes 32-63 get lanes 0-31's x.
  // r[1]: lanes 0-31 get lanes 32-63's x, lanes 32-63 keep x.
  const int upper = (threadIdx.x & 32) != 0;
  return __uint_as_float(upper ? r[0] : r[1]);
}

}  // namespace ga

namespace ga {

// RMSNorm + partial RoPE of one row chunk held in registers. Rows occupy
// aligned groups of LPR = D/8 lanes; lane c of a group holds elements
// [8c, 8c+8) in x. ``w`` points at the 8 norm weights of that chunk, or is
// null (no norm); ``rot`` = 0 skips RoPE.
// ``cs_row`` (optional) holds (cos, sin) for pair index t of this row's
// position; otherwise they are computed from ``inv_freq``.
template <int D, typename FreqT>
__device__ __forceinline__ void norm_rope_chunk(float x[8], int c, const float* w, float eps, int rot,
                                                int pos, const FreqT& inv_freq, const float2* cs_row) {
  constexpr int LPR = D / 8;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
  ss = group_sum<LPR>(ss);
  if (w) {
    const float inv = rsqrtf(ss * (1.0f / D) + eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = x[j] * inv * w[j];
  }
  if (rot > 0) {
    const int half = rot >> 1;
    const bool first = c * 8 < half;
    const bool rotated = c * 8 < rot;
    const int lane = threadIdx.x & 63;
    const int src = first ? lane + half / 8 : lane - half / 8;
    float xp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xp[j] = __shfl(x[j], rotated ? src : lane, 64);
    if (rotated) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = (first ? c * 8 : c * 8 - half) + j;
        float cs, sn;
        if (cs_row) {
          const float2 e = cs_row[t];
          cs = e.x;
          sn = e.y;
        } else {
          const float2 e = rope_cos_sin_call(pos, inv_freq[t]);
          cs = e.x;
          sn = e.y;
        }
        x[j] = first ? (x[j] * cs - xp[j] * sn) : (x[j] * cs + xp[j] * sn);
      }
    }
  }
}

__device__ __forceinline__ void unpack8(const u32x4_t raw, float x[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = lo_bf16(raw[j]);
    x[2 * j + 1] = hi_bf16(raw[j]);
  }
}

__device__ __forceinline__ u32x4_t pack8(const float x[8]) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
  return r;
}

}  // namespace ga
