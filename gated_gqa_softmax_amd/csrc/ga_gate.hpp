// Gate variants and the per-head output norm of the extended epilogues
// (device side). Sources, "Gated Attention for Large Language Models ...
// 论文阅读": sections "五个门控位置与训练结果总览" (additive Y + act(z); sigmoid
// against SiLU), "实验规模与参数预算怎样控制" (a gate shared by the heads),
// "第一条机制线索：value 与输出投影之间的非线性" (per-head RMSNorm of the attention
// output; the additive gate without its SiLU; a gate that does not depend on
// the input) and "第二条机制线索：当前 query 决定的稀疏过滤" (NS-sigmoid
// 0.5 + 0.5 sigmoid(z)).
#pragma once

#include "ga_common.hpp"
#include "ga_internal.hpp"

namespace ga {

// act(z): 0 sigmoid, 1 NS-sigmoid, 2 SiLU, 3 identity.
__device__ __forceinline__ float gate_act_f32(float z, int act) {
  if (act == 3) return z;
  const float s = sigmoid_f32(z);
  return act == 0 ? s : (act == 1 ? __builtin_fmaf(0.5f, s, 0.5f) : z * s);
}

__device__ __forceinline__ float gate_combine_f32(float y, float g, int add) { return add ? y + g : y * g; }

// Offset of the gate logits of output row ``row`` = (b*n + i)*H + h.
__device__ __forceinline__ long ext_gate_offset(const GateEpi& ge, long row, int H) {
  const long t = row / H;
  return t * ge.gts + (row - t * H) * ge.ghs;
}

// One 8-value piece (elements 8c .. 8c+7) of an output row whose D/8 pieces
// sit in D/8 consecutive lanes (every lane of the group active): the
// per-head output RMSNorm over the whole row, then combine(y, act(z)) with
// the piece's elementwise logits ``graw`` or the row's headwise logit.
template <int D>
__device__ __forceinline__ void ext_epilogue8(float (&y)[8], const GateEpi& ge, int c, u32x4_t graw,
                                              uint16_t ghead) {
  constexpr int LPR = D / 8;
  if (ge.onorm_w) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += y[j] * y[j];
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss * (1.0f / D) + ge.onorm_eps);
    const f32x4_t w0 = *(const f32x4_t*)(ge.onorm_w + c * 8);
    const f32x4_t w1 = *(const f32x4_t*)(ge.onorm_w + c * 8 + 4);
    const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = y[j] * r * wv[j];
  }
  if (ge.mode == 2) {
    float z[8];
    unpack8(graw, z);
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = gate_combine_f32(y[j], gate_act_f32(z[j], ge.act), ge.add);
  } else if (ge.mode == 1) {
    const float gv = gate_act_f32(bf16_bits_to_f32(ghead), ge.act);
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = gate_combine_f32(y[j], gv, ge.add);
  }
}

}  // namespace ga
