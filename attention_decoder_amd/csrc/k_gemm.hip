// Dequant-to-LDS fp16 MFMA GEMM for prompt prefill on gfx950.
//
// Y[m, n] = sum_k X[m, k] * f16(q[n, k] * s + bias) with MLX affine weights (TensorFold issue
// #1491, "Checkpoint handling"). The dequantised weight is rounded once to fp16 as it is staged in
// LDS; X is the fp16 activation; products accumulate in fp32 on v_mfma_f32_32x32x16_f16.
//
// Tile 128 (M) x 128 (N) x 64 (K), 256 threads as 2 x 2 waves of 64 x 64 (2 x 2 MFMA tiles).
// One LDS buffer per operand with a register prefetch of the next K tile. SwiGLU tiles interleave
// 32 gate rows and the 32 matching up rows so a lane holds both for the same output column.
#include "kernels.h"

namespace lfm3 {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSK = BK + 8;  // padded row stride (elements): 144 B rows spread the banks

template <int BITS> struct GQ { static constexpr int BYTES = 32 * BITS / 8; };

// 32 codes starting at code index 0 of `src` (a 32-code run aligned to the bit stream).
template <int BITS> LFM3_DEV void load_codes(const uint8_t* src, uint32_t (&w)[8]) {
  if constexpr (BITS == 4) {
    const uint4 v = *(const uint4*)src;
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 6) {
    const uint2* p = (const uint2*)src;
    const uint2 a = p[0], b = p[1], c = p[2];
    w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y; w[4] = c.x; w[5] = c.y;
  } else {
    const uint4 a = ((const uint4*)src)[0], b = ((const uint4*)src)[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
}

template <int BITS> LFM3_DEV uint32_t code_j(const uint32_t (&w)[8], int j) {
  if constexpr (BITS == 4) return (w[j >> 3] >> (4 * (j & 7))) & 15u;
  else if constexpr (BITS == 8) return (w[j >> 2] >> (8 * (j & 3))) & 255u;
  else {
    const int bit = 6 * j, d = bit >> 5, sh = bit & 31;
    uint32_t v = w[d] >> sh;
    if (sh > 26) v |= w[d + 1] << (32 - sh);
    return v & 63u;
  }
}

template <int BITS, int EPI>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) f16_t As[BM * LDSK];
  __shared__ __attribute__((aligned(16))) f16_t Bs[BN * LDSK];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * BM;
  const int K = a.w.k, N = a.w.n, M = a.m;
  const int half = N / 2;

  // B-tile row handled by this thread for dequant: row tid/2, codes [32*(tid&1), +32) of the tile.
  const int brow = tid >> 1, bhalf = tid & 1;
  int wrow;
  if (EPI == GEMM_SWIGLU) {
    const int out0 = blockIdx.y * 64;
    const int q = brow >> 5, r = brow & 31;
    wrow = (q & 1 ? half : 0) + out0 + (q >> 1) * 32 + r;
  } else {
    wrow = blockIdx.y * BN + brow;
  }
  const bool wvalid = wrow < N;
  const size_t row_bytes = (size_t)K * BITS / 8;
  const uint8_t* wsrc = a.w.q + (size_t)(wvalid ? wrow : 0) * row_bytes;
  const int ngr = K / a.w.group;

  uint4 areg[4];
  uint32_t wraw[8];
  float wsc = 0.f, wbi = 0.f;

  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 3, c8 = idx & 7;
      const int m = m0 + r;
      areg[i] = m < M ? *(const uint4*)(a.x + (size_t)m * a.ldx + k0 + 8 * c8) : make_uint4(0, 0, 0, 0);
    }
    const int kc = k0 + 32 * bhalf;
    if (wvalid) {
      load_codes<BITS>(wsrc + (size_t)kc * BITS / 8, wraw);
      const int g = kc / a.w.group;
      wsc = bf2f(a.w.scales[(size_t)wrow * ngr + g]);
      wbi = bf2f(a.w.biases[(size_t)wrow * ngr + g]);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 3, c8 = idx & 7;
      *(uint4*)(As + r * LDSK + 8 * c8) = areg[i];
    }
    uint32_t pk[16];
    if (wvalid) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float v0 = fmaf((float)code_j<BITS>(wraw, 2 * j), wsc, wbi);
        const float v1 = fmaf((float)code_j<BITS>(wraw, 2 * j + 1), wsc, wbi);
        pk[j] = pack_h2(v0, v1);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) pk[j] = 0;
    }
    uint4* dst = (uint4*)(Bs + brow * LDSK + 32 * bhalf);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
  };

  f32x16_v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = K / BK;
  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      f16x8_v av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + (lane & 31);
        av[i] = *(const f16x8_v*)(As + r * LDSK + 16 * ks + 8 * (lane >> 5));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 64 * wn + 32 * j + (lane & 31);
        bv[j] = *(const f16x8_v*)(Bs + r * LDSK + 16 * ks + 8 * (lane >> 5));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      sstore();
      __syncthreads();
    }
  }

  // epilogue: acc[i][j][v] is row 64wm + 32i + 8(v/4) + 4(lane/32) + v%4, col 64wn + 32j + lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row >= M) continue;
      if (EPI == GEMM_SWIGLU) {
        const int col = blockIdx.y * 64 + 32 * wn + (lane & 31);
        const float g = acc[i][0][v], u = acc[i][1][v];
        a.y[(size_t)row * a.ldy + col] = f2h_sep(g / (1.f + __expf(-g)) * u);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = blockIdx.y * BN + 64 * wn + 32 * j + (lane & 31);
          if (col < N) a.yf[(size_t)row * a.ldy + col] = acc[i][j][v];
        }
      }
    }
  }
}

template <int BITS>
static hipError_t launch_bits(hipStream_t s, const GemmArgs& a) {
  const int gm = (a.m + BM - 1) / BM;
  if (a.epi == GEMM_SWIGLU) {
    const int gn = (a.w.n / 2) / 64;
    hipLaunchKernelGGL((k_gemm<BITS, GEMM_SWIGLU>), dim3(gm, gn), dim3(256), 0, s, a);
  } else {
    const int gn = (a.w.n + BN - 1) / BN;
    hipLaunchKernelGGL((k_gemm<BITS, GEMM_STORE>), dim3(gm, gn), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(hipStream_t s, const GemmArgs& a) {
  if (a.m <= 0) return hipSuccess;
  switch (a.w.bits) {
    case 4: return launch_bits<4>(s, a);
    case 6: return launch_bits<6>(s, a);
    case 8: return launch_bits<8>(s, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lfm3
