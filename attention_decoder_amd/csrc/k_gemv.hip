// Fused dequant-GEMV for decode (batch 1..8) on gfx950.
//
// y[b, n] = sum_k x[b, k] * (q[n, k] * s[n, g] + bias[n, g]) with MLX affine weights (TensorFold
// issue #1491, "Checkpoint handling"). The weights are never rounded: per lane chunk of one group,
//   sum_k x_k (q_k s + bias) = s * sum_k x_k q_k + bias * sum_k x_k,
// where q_k enters an fp16 dot2 exactly as 1024 + q (exponent 2^10 with q in the 10-bit mantissa,
// built by one and-or per pair for every code width) and s * 1024 * sum x is subtracted.
// x is fp16; accumulation is fp32.
//
// Layout: a wave owns a group of 4 rows (SwiGLU: 2 gate rows + the 2 matching up rows); lane l
// streams chunks l, l+64, ... of each row (16 B of codes: 32 4-bit or 16 8-bit codes; 12 B of
// 6-bit codes) and the chunk's scale/bias; x is staged once per block in LDS in the pair order the
// unpacked codes come in, with per-chunk sums of x.
#include "kernels.h"

namespace lfm3 {

template <int BITS> struct QT;
template <> struct QT<4> { static constexpr int CH = 32, NDW = 4, NP = 16; };
template <> struct QT<6> { static constexpr int CH = 16, NDW = 3, NP = 8; };
template <> struct QT<8> { static constexpr int CH = 16, NDW = 4, NP = 8; };
constexpr float kMagicOff = 1024.f;       // fp16 0x6400 | q == 1024 + q for q < 1024
constexpr uint32_t kMagic2 = 0x64006400u;

// Position of code kk of a chunk inside the chunk's fp16 pair stream.
template <int BITS> LFM3_DEV int pair_pos(int kk) {
  if (BITS == 4) {
    // dword d holds codes 8d..8d+7 as nibbles; pair 4d+j = (code 8d+j, code 8d+j+4)
    const int d = kk >> 3, j = kk & 7;
    return 8 * d + (j < 4 ? 2 * j : 2 * (j - 4) + 1);
  }
  if (BITS == 8) {
    // dword d holds codes 4d..4d+3 as bytes; pair 2d = (4d, 4d+2), pair 2d+1 = (4d+1, 4d+3)
    const int d = kk >> 2, j = kk & 3;
    return 4 * d + (j == 0 ? 0 : j == 1 ? 2 : j == 2 ? 1 : 3);
  }
  return kk;  // 6-bit: pairs of consecutive codes
}

template <int BITS> LFM3_DEV void unpack(const uint32_t (&w)[QT<BITS>::NDW], uint32_t (&p)[QT<BITS>::NP]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[4 * d + j] = ((w[d] >> (4 * j)) & 0x000F000Fu) | kMagic2;
  } else if constexpr (BITS == 6) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t c[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bit = 6 * (2 * i + h);
        const int d = bit >> 5, sh = bit & 31;
        uint32_t v = w[d] >> sh;
        if (sh > 26) v |= w[d + 1] << (32 - sh);
        c[h] = v & 63u;
      }
      p[i] = (c[0] | (c[1] << 16)) | kMagic2;
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      p[2 * d] = (w[d] & 0x00FF00FFu) | kMagic2;
      p[2 * d + 1] = ((w[d] >> 8) & 0x00FF00FFu) | kMagic2;
    }
  }
}

LFM3_DEV float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_v, a), __builtin_bit_cast(f16x2_v, b), c, false);
}

template <int BITS, int BT, int EPI>
__global__ void __launch_bounds__(256) k_gemv(GemvArgs a) {
  using Q = QT<BITS>;
  extern __shared__ uint32_t smem[];
  const int K = a.w.k;
  const int NC = K / Q::CH;
  uint16_t* xp = (uint16_t*)smem;                 // [BT][K] fp16 in pair order
  float* xsum = (float*)(smem + (BT * K) / 2);    // [BT][NC]
  for (int i = threadIdx.x; i < BT * K; i += blockDim.x) {
    const int b = i / K, k = i - b * K;
    const uint16_t v = b < a.batch ? a.x[(size_t)b * a.ldx + k] : (uint16_t)0;
    const int c = k / Q::CH, kk = k - c * Q::CH;
    xp[b * K + c * Q::CH + pair_pos<BITS>(kk)] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < BT * NC; i += blockDim.x) {
    const int b = i / NC, c = i - b * NC;
    const uint16_t* p = xp + b * K + c * Q::CH;
    float s = 0.f;
    for (int j = 0; j < Q::CH; ++j) s += h2f(p[j]);
    xsum[i] = s;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = a.w.n;
  const int half = N / 2;
  const int n_groups = EPI == GEMV_SWIGLU ? half / 2 : (N + 3) / 4;
  const size_t row_bytes = (size_t)K * BITS / 8;
  const int ngr = K / a.w.group;
  uint64_t best[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) best[b] = 0;

  for (int g = blockIdx.x * 4 + wave; g < n_groups; g += gridDim.x * 4) {
    int rows[4];
    if (EPI == GEMV_SWIGLU) {
      rows[0] = 2 * g; rows[1] = 2 * g + 1; rows[2] = half + 2 * g; rows[3] = half + 2 * g + 1;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) rows[r] = min(4 * g + r, N - 1);
    }
    float acc[4][BT];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;

    for (int c = lane; c < NC; c += 64) {
      uint32_t wp[4][Q::NP];
      float sc[4], bi[4];
      const int grp = (c * Q::CH) / a.w.group;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t* src = (const uint32_t*)(a.w.q + (size_t)rows[r] * row_bytes + (size_t)c * (Q::CH * BITS / 8));
        uint32_t raw[Q::NDW];
        if constexpr (Q::NDW == 4) {
          const uint4 v = *(const uint4*)src;
          raw[0] = v.x; raw[1] = v.y; raw[2] = v.z; raw[3] = v.w;
        } else {
#pragma unroll
          for (int d = 0; d < Q::NDW; ++d) raw[d] = src[d];
        }
        unpack<BITS>(raw, wp[r]);
        sc[r] = bf2f(a.w.scales[(size_t)rows[r] * ngr + grp]);
        bi[r] = bf2f(a.w.biases[(size_t)rows[r] * ngr + grp]);
      }
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        uint32_t xv[Q::NP];
        const uint4* xs4 = (const uint4*)(xp + b * K + c * Q::CH);
#pragma unroll
        for (int q = 0; q < Q::NP / 4; ++q) {
          const uint4 v = xs4[q];
          xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
        }
        const float X = xsum[b * NC + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float d = 0.f;
#pragma unroll
          for (int p = 0; p < Q::NP; ++p) d = dot2(wp[r][p], xv[p], d);
          acc[r][b] += fmaf(sc[r], d - kMagicOff * X, bi[r] * X);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = warp_sum(acc[r][b]);

    if (lane == 0) {
      if (EPI == GEMV_STORE) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int b = 0; b < BT; ++b)
            if (b < a.batch && 4 * g + r < N) a.yf[(size_t)b * a.ldy + 4 * g + r] = acc[r][b];
      } else if (EPI == GEMV_SWIGLU) {
        // silu(a) * b is rounded to fp32, then to fp16, in every batch-size instance, so a row's
        // result does not depend on the batch it is decoded in
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            if (b >= a.batch) continue;
            const float gt = acc[j][b], up = acc[2 + j][b];
            const float sv = gt / (1.f + __expf(-gt)) * up;
            a.y[(size_t)b * a.ldy + 2 * g + j] = f2h_sep(sv);
          }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 4 * g + r;
          if (n >= N) continue;
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            if (b >= a.batch) continue;
            if (a.logits) a.logits[(size_t)b * a.ld_logits + n] = acc[r][b];
            const uint64_t key = ((uint64_t)order_key(acc[r][b]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)n);
            best[b] = key > best[b] ? key : best[b];
          }
        }
      }
    }
  }
  if (EPI == GEMV_LOGITS && lane == 0) {
#pragma unroll
    for (int b = 0; b < BT; ++b)
      if (b < a.batch && best[b]) atomicMax((unsigned long long*)&a.keys[b], (unsigned long long)best[b]);
  }
}

template <int BITS, int BT>
static hipError_t launch_bt(hipStream_t s, const GemvArgs& a) {
  using Q = QT<BITS>;
  const int K = a.w.k;
  const size_t lds = (size_t)BT * K * 2 + (size_t)BT * (K / Q::CH) * 4;
  const int N = a.w.n;
  const int n_groups = a.epi == GEMV_SWIGLU ? N / 4 : (N + 3) / 4;
  int grid = (n_groups + 3) / 4;
  if (grid > 2048) grid = 2048;
  switch (a.epi) {
    case GEMV_STORE: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE>), dim3(grid), dim3(256), lds, s, a); break;
    case GEMV_SWIGLU: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_SWIGLU>), dim3(grid), dim3(256), lds, s, a); break;
    default: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_LOGITS>), dim3(grid), dim3(256), lds, s, a); break;
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_bits(hipStream_t s, const GemvArgs& a) {
  using Q = QT<BITS>;
  const int K = a.w.k;
  auto lds_for = [&](int bt) { return (size_t)bt * K * 2 + (size_t)bt * (K / Q::CH) * 4; };
  int bt = a.batch <= 1 ? 1 : a.batch <= 2 ? 2 : a.batch <= 4 ? 4 : 8;
  while (bt > 1 && lds_for(bt) > 65536) bt >>= 1;
  if (a.batch > bt) {
    // split the batch into launches that fit the 64 KiB of LDS
    for (int b0 = 0; b0 < a.batch; b0 += bt) {
      GemvArgs p = a;
      p.batch = a.batch - b0 < bt ? a.batch - b0 : bt;
      p.x = a.x + (size_t)b0 * a.ldx;
      if (p.y) p.y = a.y + (size_t)b0 * a.ldy;
      if (p.yf) p.yf = a.yf + (size_t)b0 * a.ldy;
      if (p.logits) p.logits = a.logits + (size_t)b0 * a.ld_logits;
      if (p.keys) p.keys = a.keys + b0;
      hipError_t e = launch_bits<BITS>(s, p);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  switch (bt) {
    case 1: return launch_bt<BITS, 1>(s, a);
    case 2: return launch_bt<BITS, 2>(s, a);
    case 4: return launch_bt<BITS, 4>(s, a);
    default: return launch_bt<BITS, 8>(s, a);
  }
}

hipError_t launch_gemv(hipStream_t s, const GemvArgs& a) {
  if (a.batch <= 0) return hipSuccess;
  switch (a.w.bits) {
    case 4: return launch_bits<4>(s, a);
    case 6: return launch_bits<6>(s, a);
    case 8: return launch_bits<8>(s, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lfm3
