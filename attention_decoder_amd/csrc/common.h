// Shared device-side types and helpers of the gfx950 LFM3 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define LFM3_DEV __device__ __forceinline__
#define LFM3_HOST_DEV __host__ __device__ __forceinline__

typedef uint16_t bf16_t;  // bf16 bit pattern (the stored scales and biases, norm and conv weights)
typedef uint16_t f16_t;   // IEEE fp16 bit pattern (matmul operands, KV cache, conv state)
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_v;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_v;
typedef __attribute__((ext_vector_type(16))) float f32x16_v;

namespace lfm3 {

constexpr int kMaxBatch = 64;
// Argmax partials of the head: block p of a logits launch stores its best key of row r at
// keys[r * kArgmaxParts + p] (plain stores: no atomics on a shared word); the finalize takes the
// max over all parts of a row and clears them, so unwritten parts read zero.
constexpr int kArgmaxParts = 1024;
constexpr int kHeadDim = 128;
constexpr int kHalfDim = 64;
constexpr int kQPerKv = 4;
constexpr int kPageTokens = 16;
constexpr int kMaxTaps = 8;

// Which slot and position each row of a pass belongs to. A prefill pass is one slot at
// consecutive positions (mode 0); a decode step is one row per slot (mode 1).
struct Rows {
  int32_t n;
  int32_t mode;
  int32_t slot0;
  int32_t pos0;
  int32_t slot[kMaxBatch];
  int32_t pos[kMaxBatch];
};

LFM3_DEV int row_slot(const Rows& r, int i) { return r.mode == 0 ? r.slot0 : r.slot[i]; }
LFM3_DEV int row_pos(const Rows& r, int i) { return r.mode == 0 ? r.pos0 + i : r.pos[i]; }

LFM3_DEV float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16, round to nearest even (NaN kept quiet).
LFM3_DEV bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

LFM3_DEV float h2f(f16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
// float -> fp16, round to nearest even (the hardware conversion).
LFM3_DEV f16_t f2h(float f) { return __builtin_bit_cast(f16_t, (_Float16)f); }
LFM3_DEV uint32_t pack_h2(float lo, float hi) { return (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16); }
// float -> fp16 (RNE) that the compiler cannot fuse with the multiply producing `f` (it would
// otherwise pick a single-rounding mixed FMA in some template instances and not in others).
LFM3_DEV f16_t f2h_sep(float f) {
  uint32_t r;
  asm("v_cvt_f16_f32 %0, %1" : "=v"(r) : "v"(f));
  return (f16_t)(r & 0xffffu);
}

// a - b, rounded once, that the compiler cannot contract with the multiply producing `a` (the
// fp16 remainder x - f16(x) must be the same value in every kernel that forms it).
LFM3_DEV float sub_sep(float a, float b) {
  float r;
  asm("v_sub_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

LFM3_DEV float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
LFM3_DEV float warp_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// DPP lane moves: quad_perm [1,0,3,2] (0xb1), [2,3,0,1] (0x4e), row_half_mirror (0x141),
// row_mirror (0x140).
template <int CTRL> LFM3_DEV float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Sum over each 16-lane row, returned in every lane of the row.
LFM3_DEV float row16_sum(float v) {
  v += dpp_mov<0xb1>(v);
  v += dpp_mov<0x4e>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}
LFM3_DEV float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Sum over the 64 lanes of a wave in a fixed order; the result is wave-uniform.
LFM3_DEV float wave_sum(float v) {
  const float s = row16_sum(v);
  return ((readlane_f(s, 0) + readlane_f(s, 16)) + readlane_f(s, 32)) + readlane_f(s, 48);
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024); `red` holds >= 16 floats of LDS.
LFM3_DEV float block_sum(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Orderable key for a float: larger float -> larger key; NaN ranks as -inf.
LFM3_DEV uint32_t order_key(float f) {
  if (f != f) f = -__builtin_huge_valf();
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Storage formats of a linear's weight.
enum WeightFmt {
  FMT_AFFINE = 0,   // MLX affine: `bits`-bit codes, bf16 scale and bias per `group` along K
  FMT_BF16 = 1,     // stored bf16 values
  FMT_NVFP4 = 2,    // e2m1 codes (two a byte, element 2i in the low nibble), an e4m3 scale per 16 k, an fp32 tensor scale
  FMT_FP8B = 3      // e4m3 codes, an fp32 scale per 128 x 128 block
};

// A linear [N, K] as stored in the blob (device pointers into it).
struct QLinear {
  const uint8_t* q;       // affine: [N, K * bits / 8]; bf16: [N, K] bf16; nvfp4: [N, K / 2]; fp8b: [N, K]
  const bf16_t* scales;   // affine: [N, K / group]
  const bf16_t* biases;   // affine: [N, K / group]
  int32_t n, k, bits, group;
  int32_t fmt;            // WeightFmt
  const uint8_t* bscale;  // nvfp4: e4m3 [N, K / 16]; fp8b: fp32 [ceil(N / 128), ceil(K / 128)]
  float tscale;           // nvfp4: the tensor scale (1 otherwise)
};

// FP4 E2M1 code (4 bits) as an fp16 bit pattern worth 2^-14 of its value: the exponent and mantissa
// bits moved to fp16 bits 11..9 (exponent 0 becomes an fp16 subnormal, as E2M1's is), the sign to 15.
LFM3_HOST_DEV uint32_t e2m1_f16_scaled(uint32_t c) { return ((c & 7u) << 9) | ((c & 8u) << 12); }
// FP8 E4M3 byte as an fp16 bit pattern worth 2^-8 of its value (exponent and mantissa to bits
// 13..7, sign to 15; exponent 0 is a subnormal in both). NaN bytes (0x7F, 0xFF) are never stored.
LFM3_HOST_DEV uint32_t e4m3_f16_scaled(uint32_t b) { return ((b & 0x7Fu) << 7) | ((b & 0x80u) << 8); }
LFM3_DEV float e4m3_value(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)e4m3_f16_scaled(b)) * 256.f;
}
LFM3_DEV float e2m1_value(uint32_t c) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)e2m1_f16_scaled(c)) * 16384.f;
}

// Weight (n, k) of a non-affine linear in fp32: exact for bf16; for nvfp4 and fp8b the code times
// its block scale is exact in fp32 and one fp32 multiply rounds the product with the tensor scale
// (nvfp4) or the fp32 block scale (fp8b).
LFM3_DEV float weight_value(const QLinear& w, int n, int k) {
  if (w.fmt == FMT_BF16) {
    const uint16_t b = ((const uint16_t*)w.q)[(size_t)n * w.k + k];
    return __uint_as_float((uint32_t)b << 16);
  }
  if (w.fmt == FMT_NVFP4) {
    const uint32_t byte = w.q[(size_t)n * (w.k / 2) + k / 2];
    const uint32_t c = (k & 1) ? byte >> 4 : byte & 15u;
    const float sc = e4m3_value(w.bscale[(size_t)n * (w.k / 16) + k / 16]);
    return (e2m1_value(c) * sc) * w.tscale;
  }
  const int kb = (w.k + 127) / 128;
  const float sc = ((const float*)w.bscale)[(size_t)(n / 128) * kb + k / 128];
  return e4m3_value(w.q[(size_t)n * w.k + k]) * sc;
}

}  // namespace lfm3
