// Merge of attention partials computed over disjoint KV ranges: device code.
//
// A partial for KV range g is O_g = Σ_{j∈g} e^{s_j - lse_g} v_j (normalised
// within the range) and lse_g = ln Σ_{j∈g} e^{s_j}.  Softmax attention over
// the union follows from the associativity of the (max, sum, output) carrier
// ("Learning FlashAttention the Hard Way - Part 2", "Wrap-Up": the schedule
// needs only associativity; its references name split-KV as the split-K of
// that monoid, and "The Move Stack" combines per-CTA partial reductions with a
// separate kernel):
//     lse = ln Σ_g e^{lse_g},   O = Σ_g e^{lse_g - lse} O_g.
// A range with no keys has lse_g = -inf and weight 0.
//
// HBM-bound elementwise work: each thread owns 8 consecutive head-dim entries
// of one query row, reads them from every partial with 16-byte loads and writes
// the merged row once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_kernel.h"

namespace attn {

struct MergeParams {
  const float* o_parts;    // n_parts consecutive contiguous [B, H, S, D] fp32 arrays
  const float* lse_parts;  // n_parts consecutive contiguous [B, H, S] fp32 arrays
  void* o;                 // output, element type T, strides below (D contiguous)
  float* lse;              // contiguous [B, H, S]; may be null
  long long o_sb, o_sh;    // output batch and head strides (elements)
  int o_ss;                // output row stride (elements)
  int n_parts;
  int H, S;
  long long rows;          // B * H * S
  long long part_stride;   // B * H * S * D
  int f32_out;             // 1: o is fp32 (else the 16-bit type T)
};

template <class T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 8;              // threads per row
  constexpr int RPB = 256 / TPR;          // rows per workgroup
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= p.rows) return;
  const int d0 = (threadIdx.x % TPR) * 8;

  float mx = -__builtin_inff();
  for (int g = 0; g < p.n_parts; ++g) mx = fmaxf(mx, p.lse_parts[g * p.rows + row]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (mx != -__builtin_inff()) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float* src = p.o_parts + row * D + d0;
    for (int g = 0; g < p.n_parts; ++g) {
      const float w = __builtin_amdgcn_exp2f((p.lse_parts[g * p.rows + row] - mx) * kLog2e);
      const float4 a = *reinterpret_cast<const float4*>(src + g * p.part_stride);
      const float4 b = *reinterpret_cast<const float4*>(src + g * p.part_stride + 4);
      acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
      acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
      den += w;
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const long long bh = row / p.S;
  const int s = (int)(row - bh * p.S);
  const int b = (int)(bh / p.H), h = (int)(bh - (long long)b * p.H);
  const long long off = b * p.o_sb + h * p.o_sh + (long long)s * p.o_ss + d0;
  if (p.f32_out) {
    float* dst = static_cast<float*>(p.o) + off;
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = Mma<T>::pack(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    uint4 v4 = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.o) + off) = v4;
  }
  if (p.lse != nullptr && d0 == 0)
    p.lse[row] = den > 0.f ? mx + __builtin_amdgcn_logf(den) * 0.69314718055994531f : -__builtin_inff();
}

}  // namespace attn
