// Vectorised residual + RMSNorm of one hidden row, shared by k_resid_norm and the decode GEMV's
// norm prologue so that the fused and unfused forms give bitwise the same values.
//
// "LFM3-1.7B port" (TensorFold issue #1491), layer structure: sandwich RMSNorms, eps inside the
// square root, the weight multiplying directly:
//   h_new = h + rmsnorm(m) * w_post   (m absent: h_new = h)
//   x     = rmsnorm(h_new) * w_pre
// Element layout: thread t of a 256-thread block owns the 8-element vectors v = t + 256 j
// (j < kVecBlocks), i.e. elements [8v, 8v + 8) of the row; K % 8 == 0 and K <= 4096.
// Every sum runs in a fixed order: per thread j-major then element order (fmaf), then the wave
// (fixed DPP tree), then the four waves in wave order.
#pragma once
#include "common.h"

namespace lfm3 {

constexpr int kVecBlocks = 2;

LFM3_DEV void load_f32x8(const float* p, float (&o)[8]) {
  const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
LFM3_DEV void store_f32x8(float* p, const float (&o)[8]) {
  ((float4*)p)[0] = make_float4(o[0], o[1], o[2], o[3]);
  ((float4*)p)[1] = make_float4(o[4], o[5], o[6], o[7]);
}
// 8 raw 16-bit values (bf16 or fp16 bits) as one 16-byte load.
LFM3_DEV uint4 load_u16x8(const uint16_t* p) { return *(const uint4*)p; }
LFM3_DEV void bf16x8_to_f32(const uint4 u, float (&o)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Sum over the 256 threads of a block; `red` holds 4 floats of LDS per call site. Ends with a
// barrier-free read: the caller separates reuses of `red` with __syncthreads().
LFM3_DEV float block_sum4(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

}  // namespace lfm3
