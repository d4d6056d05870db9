// Dequant-to-LDS fp16 MFMA GEMM for prompt prefill on gfx950.
//
// Y[m, n] = sum_k X[m, k] * f16(q[n, k] * s + bias) with MLX affine weights (TensorFold issue
// #1491, "Checkpoint handling"). The dequantised weight is rounded once to fp16 as it is staged in
// LDS; X is the fp16 activation; products accumulate in fp32 on v_mfma_f32_32x32x16_f16.
//
// Block tile BM = 128 rows of X by BN = 256 (or 128) weight rows by BK = 64, four waves as 2 x 2,
// each wave 64 x BN/2 (2 x BN/64 MFMA tiles of 32 x 32). One LDS buffer per operand; the next K
// tile's global loads are issued before the current tile's MFMAs (register prefetch), and two
// blocks share a CU so that one block's staging overlaps the other's MFMAs.
//
// Dequant in packed fp16: a code pair becomes (1024 + q0, 1024 + q1) with one and-or (the fp16
// bit pattern 0x6400 | q), 1024 is subtracted exactly, and one packed fp16 FMA forms q * s + b
// with a single rounding. The pairs come out in a fixed order within each 8-code group; X is
// staged in LDS with the same order, which leaves every dot product unchanged.
//
// Loads are branch-free (rows past M or N read a clamped valid row whose results are not stored).
// SwiGLU tiles interleave 32 gate rows and the 32 matching up rows, so a lane holds both halves of
// an output column.
#include "kernels.h"

namespace lfm3 {

constexpr int BM = 128, BK = 64;
constexpr int LDSK = BK + 8;  // padded row stride (elements): 144-byte rows keep ds_read_b128 conflict-free

// Order of 8 consecutive k inside the staged tiles (per 16-byte group), matching the pair order of
// the dequant: 4-bit (0,4)(1,5)(2,6)(3,7); 8-bit (0,2)(1,3)(4,6)(5,7); 6-bit natural.
template <int BITS> LFM3_DEV u32x4_v perm8(u32x4_v h) {
  if constexpr (BITS == 4) {
    return u32x4_v{__builtin_amdgcn_perm(h[2], h[0], 0x05040100u), __builtin_amdgcn_perm(h[2], h[0], 0x07060302u),
                   __builtin_amdgcn_perm(h[3], h[1], 0x05040100u), __builtin_amdgcn_perm(h[3], h[1], 0x07060302u)};
  } else if constexpr (BITS == 8) {
    return u32x4_v{__builtin_amdgcn_perm(h[1], h[0], 0x05040100u), __builtin_amdgcn_perm(h[1], h[0], 0x07060302u),
                   __builtin_amdgcn_perm(h[3], h[2], 0x05040100u), __builtin_amdgcn_perm(h[3], h[2], 0x07060302u)};
  } else {
    return h;
  }
}

constexpr uint32_t kMagic2 = 0x64006400u;  // fp16 (1024, 1024); 0x6400 | q == 1024 + q

LFM3_DEV uint32_t deq2(uint32_t magic_pair, f16x2_v s2, f16x2_v b2) {
  const f16x2_v q = __builtin_bit_cast(f16x2_v, magic_pair) - f16x2_v{(_Float16)1024.f, (_Float16)1024.f};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
}

// Codes of one thread's run: CPT codes (64 or 32) of one weight row.
template <int BITS, int CPT> struct Codes {
  static constexpr int BYTES = CPT * BITS / 8;
  static constexpr int NV = BYTES / 16;  // 16-byte loads (q6 with 32 codes: 24 bytes, see load)
  uint32_t w[BYTES / 4];
};

template <int BITS, int CPT>
LFM3_DEV void load_codes(const uint8_t* src, Codes<BITS, CPT>& c) {
  constexpr int NW = Codes<BITS, CPT>::BYTES / 4;
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int v = 0; v < NW / 4; ++v) {
      const u32x4_v t = *(const u32x4_v*)(src + 16 * v);
      c.w[4 * v] = t[0]; c.w[4 * v + 1] = t[1]; c.w[4 * v + 2] = t[2]; c.w[4 * v + 3] = t[3];
    }
  } else {
#pragma unroll
    for (int v = 0; v < NW / 2; ++v) {
      const uint2 t = *(const uint2*)(src + 8 * v);
      c.w[2 * v] = t.x; c.w[2 * v + 1] = t.y;
    }
  }
}

// Dequantise the run into CPT fp16 (CPT / 2 words) in the tile order. `sel` picks the scale pair
// of codes at offsets >= group (two groups in a 64-code run at group 32).
template <int BITS, int CPT>
LFM3_DEV void dequant_run(const Codes<BITS, CPT>& c, const f16x2_v (&s2)[2], const f16x2_v (&b2)[2], int group,
                          uint32_t (&out)[CPT / 2]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < CPT / 8; ++d) {
      const int g = (8 * d >= group) ? 1 : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[4 * d + j] = deq2(((c.w[d] >> (4 * j)) & 0x000F000Fu) | kMagic2, s2[g], b2[g]);
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int d = 0; d < CPT / 4; ++d) {
      const int g = (4 * d >= group) ? 1 : 0;
      out[2 * d] = deq2((c.w[d] & 0x00FF00FFu) | kMagic2, s2[g], b2[g]);
      out[2 * d + 1] = deq2(((c.w[d] >> 8) & 0x00FF00FFu) | kMagic2, s2[g], b2[g]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < CPT / 2; ++i) {
      const int g = (2 * i >= group) ? 1 : 0;
      uint32_t q2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bit = 6 * (2 * i + h);
        const int d = bit >> 5, sh = bit & 31;
        uint32_t v = c.w[d] >> sh;
        if (sh > 26) v |= c.w[d + 1] << (32 - sh);
        q2[h] = v & 63u;
      }
      out[i] = deq2((q2[0] | (q2[1] << 16)) | kMagic2, s2[g], b2[g]);
    }
  }
}

LFM3_DEV f16x2_v bf16_pair(bf16_t b) {
  const _Float16 h = (_Float16)bf2f(b);
  return f16x2_v{h, h};
}

template <int BITS, int EPI, int BN>
__global__ void __launch_bounds__(256, 2) k_gemm(GemmArgs a) {
  constexpr int NJ = BN / 64;          // 32-wide MFMA column tiles per wave
  constexpr int CPT = BN == 256 ? 64 : 32;  // codes per thread per K tile
  __shared__ __attribute__((aligned(16))) f16_t As[BM * LDSK];
  __shared__ __attribute__((aligned(16))) f16_t Bs[BN * LDSK];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * BM;
  const int K = a.w.k, N = a.w.n, M = a.m;
  const int half = N / 2;

  // weight row of this thread's run: tile row brow, codes [kofs, kofs + CPT) of the K tile
  const int brow = BN == 256 ? tid : tid >> 1;
  const int kofs = BN == 256 ? 0 : 32 * (tid & 1);
  int wrow;
  if constexpr (EPI == GEMM_SWIGLU) {
    const int wpart = brow / (BN / 2), j = (brow % (BN / 2)) / 32, r = brow & 31;
    const int outc = blockIdx.y * (BN / 2) + wpart * (BN / 4) + (j >> 1) * 32 + r;
    wrow = (j & 1 ? half : 0) + outc;
  } else {
    wrow = min((int)blockIdx.y * BN + brow, N - 1);
  }
  const size_t row_bytes = (size_t)K * BITS / 8;
  const uint8_t* wsrc = a.w.q + (size_t)wrow * row_bytes;
  const int ngr = K / a.w.group;
  const int group = a.w.group;

  u32x4_v areg[4];
  Codes<BITS, CPT> creg;
  bf16_t sraw[2], braw[2];

  // K tiles 0 .. nk-1 read x; with a remainder input, tiles nk .. 2nk-1 read x_lo against the same
  // weight tiles (Y = x W + x_lo W)
  const int nk = K / BK;
  auto gload = [&](int kt) {
    const bool second = kt >= nk;
    const int k0 = (second ? kt - nk : kt) * BK;
    const f16_t* xs = second ? a.x_lo : a.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 3, c8 = idx & 7;
      const int m = min(m0 + r, M - 1);
      areg[i] = *(const u32x4_v*)(xs + (size_t)m * a.ldx + k0 + 8 * c8);
    }
    const int kc = k0 + kofs;
    load_codes<BITS, CPT>(wsrc + (size_t)kc * BITS / 8, creg);
    const int g0 = kc / group, g1 = (kc + CPT - 1) / group;
    sraw[0] = a.w.scales[(size_t)wrow * ngr + g0];
    braw[0] = a.w.biases[(size_t)wrow * ngr + g0];
    sraw[1] = a.w.scales[(size_t)wrow * ngr + g1];
    braw[1] = a.w.biases[(size_t)wrow * ngr + g1];
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 3, c8 = idx & 7;
      *(u32x4_v*)(As + r * LDSK + 8 * c8) = perm8<BITS>(areg[i]);
    }
    const f16x2_v s2[2] = {bf16_pair(sraw[0]), bf16_pair(sraw[1])};
    const f16x2_v b2[2] = {bf16_pair(braw[0]), bf16_pair(braw[1])};
    uint32_t pk[CPT / 2];
    dequant_run<BITS, CPT>(creg, s2, b2, group, pk);
    u32x4_v* dst = (u32x4_v*)(Bs + brow * LDSK + kofs);
#pragma unroll
    for (int q = 0; q < CPT / 8; ++q) dst[q] = u32x4_v{pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
  };

  f32x16_v acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nkt = a.x_lo ? 2 * nk : nk;
  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      f16x8_v av[2], bv[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + (lane & 31);
        av[i] = *(const f16x8_v*)(As + r * LDSK + 16 * ks + 8 * (lane >> 5));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = (BN / 2) * wn + 32 * j + (lane & 31);
        bv[j] = *(const f16x8_v*)(Bs + r * LDSK + 16 * ks + 8 * (lane >> 5));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nkt) {
      sstore();
      __syncthreads();
    }
  }

  // epilogue: acc[i][j][v] is row 64wm + 32i + 8(v/4) + 4(lane/32) + v%4, tile column
  // (BN/2) wn + 32 j + lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row >= M) continue;
      if constexpr (EPI == GEMM_SWIGLU) {
#pragma unroll
        for (int jj = 0; jj < NJ / 2; ++jj) {
          const int col = blockIdx.y * (BN / 2) + wn * (BN / 4) + 32 * jj + (lane & 31);
          const float g = acc[i][2 * jj][v], u = acc[i][2 * jj + 1][v];
          a.y[(size_t)row * a.ldy + col] = f2h_sep(g / (1.f + __expf(-g)) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = blockIdx.y * BN + (BN / 2) * wn + 32 * j + (lane & 31);
          if (col < N) a.yf[(size_t)row * a.ldy + col] = acc[i][j][v];
        }
      }
    }
  }
}

template <int BITS, int BN>
static void launch_bn(hipStream_t s, const GemmArgs& a) {
  const int gm = (a.m + BM - 1) / BM;
  if (a.epi == GEMM_SWIGLU) {
    hipLaunchKernelGGL((k_gemm<BITS, GEMM_SWIGLU, BN>), dim3(gm, a.w.n / BN), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_gemm<BITS, GEMM_STORE, BN>), dim3(gm, (a.w.n + BN - 1) / BN), dim3(256), 0, s, a);
  }
}

template <int BITS>
static hipError_t launch_bits(hipStream_t s, const GemmArgs& a) {
  // wide tiles for wide weights (less re-reading of X); 128-wide for the 2048-row ones, which
  // would otherwise leave half the chip idle
  const bool wide = a.epi == GEMM_SWIGLU ? (a.w.n % 256 == 0 && a.w.n >= 4096) : a.w.n >= 4096;
  if (wide) launch_bn<BITS, 256>(s, a);
  else launch_bn<BITS, 128>(s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(hipStream_t s, const GemmArgs& a) {
  if (a.m <= 0) return hipSuccess;
  // 16-byte rows of X, whole K tiles, whole code runs
  if (a.w.k % BK || a.ldx % 8 || (uintptr_t)a.x % 16 || (uintptr_t)a.x_lo % 16 || (a.epi == GEMM_SWIGLU && a.w.n % 128))
    return hipErrorInvalidValue;
  switch (a.w.bits) {
    case 4: return launch_bits<4>(s, a);
    case 6: return launch_bits<6>(s, a);
    case 8: return launch_bits<8>(s, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lfm3
