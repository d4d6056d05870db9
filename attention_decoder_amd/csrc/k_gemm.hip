// Dequant fp16 MFMA GEMM for prompt prefill on gfx950.
//
// Y[m, n] = sum_k X[m, k] * f16(q[n, k] * s + bias) with MLX affine weights (TensorFold issue
// #1491, "Checkpoint handling"). The dequantised weight is rounded once to fp16; X is the fp16
// activation; products accumulate in fp32 on v_mfma_f32_32x32x16_f16.
//
// Block tile BM (128 or 64) rows of X by 256 weight rows by BK = 64, four waves side by side in N:
// wave w owns weight rows [64w, 64w + 64) of the tile and every row of X, as BM/32 x 2 MFMA tiles.
// Only X goes through LDS (double-buffered, one barrier per K tile). The weights never touch LDS:
// each lane loads the codes its MFMA B operand needs (row n = lane % 32 of a 32-row tile, the 32
// consecutive k of its lane half) and dequantises them straight into operand registers, so the
// LDS traffic per MFMA is one 16-byte A read per lane. The weights are read from a re-tiled copy
// (GemmW, built once by k_repack) in which every load instruction of a wave reads whole
// contiguous 1 KB (or 512 B) runs, and the scale and bias of a lane's group come as one fp16 pair.
//
// K order inside an MFMA: for k sub-step t the lane half h supplies k = 32h + 8t .. 32h + 8t + 7 of
// the K tile, in order (the re-tiled 4-bit words hold their codes at the nibble order the
// byte-permute unpack needs), so X is staged in LDS as it is.
//
// Dequant in packed fp16: a code pair becomes (1024 + q0, 1024 + q1) with one byte permute (the
// fp16 bit pattern 0x6400 | q), 1024 is subtracted exactly, and one packed fp16 FMA forms
// q * s + b with a single rounding.
//
// Loads are branch-free (rows past M or N read a clamped valid row whose results are not stored).
// SwiGLU: a lane's two weight rows are the gate row and the matching up row of one output column.
#include <type_traits>

#include "kernels.h"

namespace lfm3 {

constexpr int BK = 64;
constexpr int LDSK = BK + 8;  // padded X row stride (elements): 144-byte rows keep ds_read_b128 conflict-free
constexpr int BN = 256;       // weight rows per block tile

constexpr uint32_t kMagic2 = 0x64006400u;  // fp16 (1024, 1024); 0x6400 | q == 1024 + q

LFM3_DEV uint32_t deq2(uint32_t magic_pair, f16x2_v s2, f16x2_v b2) {
  const f16x2_v q = __builtin_bit_cast(f16x2_v, magic_pair) - f16x2_v{(_Float16)1024.f, (_Float16)1024.f};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
}

// The 32 codes of one lane's run (one weight row, 32 consecutive k): 16, 24 or 32 bytes.
template <int BITS> struct Run {
  static constexpr int NW = BITS;  // 32 codes * BITS bits / 32
  uint32_t w[NW];
};

// Raw buffer loads: the lane's byte offset in a VGPR, the K-tile offset in an SGPR, so the loop
// carries no per-lane address arithmetic.
LFM3_DEV __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Plane layout of a lane's 32 codes in the re-tiled copy: bytes per lane per plane, planes.
template <int BITS> struct Planes {
  static constexpr int PB = BITS == 6 ? 8 : 16;
  static constexpr int NP = 4 * BITS / PB;
};

template <int BITS> LFM3_DEV void load_run(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, Run<BITS>& r) {
  constexpr int PB = Planes<BITS>::PB;
  if constexpr (BITS == 6) {
#pragma unroll
    for (int v = 0; v < 3; ++v) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(rs, voff + 64 * PB * v, soff, 0);
      r.w[2 * v] = t[0]; r.w[2 * v + 1] = t[1];
    }
  } else {
#pragma unroll
    for (int v = 0; v < BITS / 4; ++v) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 64 * PB * v, soff, 0);
      r.w[4 * v] = t[0]; r.w[4 * v + 1] = t[1]; r.w[4 * v + 2] = t[2]; r.w[4 * v + 3] = t[3];
    }
  }
}

// Byte selectors of v_perm_b32(0x64646464, t): [t.b0, 0x64, t.b1, 0x64] and [t.b2, 0x64, t.b3, 0x64],
// i.e. the fp16 pairs (1024 + t.b0, 1024 + t.b1) and (1024 + t.b2, 1024 + t.b3) for bytes < 1024.
constexpr uint32_t kSelLo = 0x04010400u, kSelHi = 0x04030402u;
constexpr uint32_t kBytes64 = 0x64646464u;

// Codes 8T .. 8T+7 of a run as the fp16 MFMA operand (4 pairs in the tile order).
template <int BITS, int T> LFM3_DEV f16x8_v deq8(const Run<BITS>& r, f16x2_v s2, f16x2_v b2) {
  uint32_t p[4];
  if constexpr (BITS == 4) {
    // nibbles 0, 2, 4, 6 (codes 0 .. 3 after the re-tiling) and 1, 3, 5, 7 (codes 4 .. 7) as bytes
    const uint32_t t0 = r.w[T] & 0x0F0F0F0Fu, t1 = (r.w[T] >> 4) & 0x0F0F0F0Fu;
    p[0] = deq2(__builtin_amdgcn_perm(kBytes64, t0, kSelLo), s2, b2);
    p[1] = deq2(__builtin_amdgcn_perm(kBytes64, t0, kSelHi), s2, b2);
    p[2] = deq2(__builtin_amdgcn_perm(kBytes64, t1, kSelLo), s2, b2);
    p[3] = deq2(__builtin_amdgcn_perm(kBytes64, t1, kSelHi), s2, b2);
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      p[2 * d] = deq2(__builtin_amdgcn_perm(kBytes64, r.w[2 * T + d], kSelLo), s2, b2);
      p[2 * d + 1] = deq2(__builtin_amdgcn_perm(kBytes64, r.w[2 * T + d], kSelHi), s2, b2);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t q2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bit = 6 * (8 * T + 2 * i + h);
        const int d = bit >> 5, sh = bit & 31;
        uint32_t v = r.w[d] >> sh;
        if (sh > 26) v |= r.w[d + 1] << (32 - sh);
        q2[h] = v & 63u;
      }
      p[i] = deq2((q2[0] | (q2[1] << 16)) | kMagic2, s2, b2);
    }
  }
  return __builtin_bit_cast(f16x8_v, u32x4_v{p[0], p[1], p[2], p[3]});
}

// BITS = 16: the weights come from the fp16 copy (GemmW::w16), already in operand order.
template <int BITS, int EPI, int BM>
__global__ void __launch_bounds__(256, 2) k_gemm(GemmArgs a) {
  constexpr bool F16 = BITS == 16;
  constexpr int QB = F16 ? 4 : BITS;             // code width of the (unused) codes path
  constexpr int MT = BM / 32;                  // 32-row MFMA tiles per wave
  constexpr int AV = BM * BK / 8 / 256;        // 16-byte X pieces per thread per K tile
  __shared__ __attribute__((aligned(16))) f16_t As[2][BM * LDSK];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, c32 = lane & 31;
  const int m0 = blockIdx.x * BM;
  const int K = a.w.k, N = a.w.n, M = a.m;

  // the lane's two weight rows (MFMA column c32 of the wave's two 32-row tiles): their tiles in the
  // re-tiled copy (past N: the last tile, whose results are not stored)
  int wtile[2], wrow0;
  if constexpr (EPI == GEMM_SWIGLU) {
    wtile[0] = blockIdx.y * (BN / 64) + wave;
    wtile[1] = (N / 2) / 32 + wtile[0];
    wrow0 = 32 * wtile[0] + c32;   // output column
  } else {
    wtile[0] = min((int)blockIdx.y * (BN / 32) + 2 * wave, a.w.ntile - 1);
    wtile[1] = min((int)blockIdx.y * (BN / 32) + 2 * wave + 1, a.w.ntile - 1);
    wrow0 = 0;
  }
  constexpr uint32_t kTileBytes = F16 ? 4096u : 256u * BITS;    // one (32-row, 64-k) tile

  // K tiles 0 .. nk-1 read x; with a remainder input, tiles nk .. 2nk-1 read x_lo against the same
  // weight tiles (Y = x W + x_lo W). With a K split, block z runs tiles [z nk/2, (z + 1) nk/2).
  const int nk = K / BK;
  const int kt0 = blockIdx.z * (nk / 2);
  const int nkt = a.yf2 ? kt0 + nk / 2 : (a.x_lo ? 2 * nk : nk);   // end of this block's tiles
  float* const yout = blockIdx.z ? a.yf2 : a.yf;

  const uint32_t xbytes = (uint32_t)((size_t)(M - 1) * a.ldx + K) * 2u;
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.x, xbytes);
  const __amdgpu_buffer_rsrc_t rxl = rsrc_of(a.x_lo ? a.x_lo : a.x, xbytes);
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(F16 ? (const void*)a.w.w16 : (const void*)a.w.codes, (uint32_t)a.w.ntile * nk * kTileBytes);
  const __amdgpu_buffer_rsrc_t rsb = rsrc_of(a.w.sb, (uint32_t)a.w.ntile * nk * 256u);

  // per-lane byte offsets, fixed over the K loop
  uint32_t xoff[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx >> 3, c8 = idx & 7;
    xoff[i] = ((uint32_t)min(m0 + r, M - 1) * (uint32_t)a.ldx + 8u * c8) * 2u;
  }
  uint32_t qoff[2], sboff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    qoff[j] = (uint32_t)wtile[j] * nk * kTileBytes + (uint32_t)lane * (F16 ? 16u : (uint32_t)Planes<QB>::PB);
    sboff[j] = ((uint32_t)wtile[j] * nk * 64u + lane) * 4u;
  }

  u32x4_v areg[AV];
  auto load_x = [&](int kt) {
    const bool second = kt >= nk;
    const uint32_t k0 = (uint32_t)(second ? kt - nk : kt) * BK;
    const __amdgpu_buffer_rsrc_t r = second ? rxl : rx;
#pragma unroll
    for (int i = 0; i < AV; ++i) areg[i] = __builtin_amdgcn_raw_buffer_load_b128(r, xoff[i], 2u * k0, 0);
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 3, c8 = idx & 7;
      *(u32x4_v*)(&As[buf][r * LDSK + 8 * c8]) = areg[i];
    }
  };
  // weight registers in two sets (even / odd K tiles), so that no value has to be copied across
  // the loop edge (a copy would make every iteration wait for the loads it just issued)
  struct WSetQ {
    Run<QB> run[2];
    uint32_t sb[2];   // fp16 (scale, bias)
  };
  struct WSet16 {
    u32x4_v p[2][4];   // the operand registers themselves
  };
  using WSet = std::conditional_t<F16, WSet16, WSetQ>;
  auto load_w = [&](int kt, WSet& w) {
    const uint32_t kk = (uint32_t)(kt >= nk ? kt - nk : kt);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (F16) {
#pragma unroll
        for (int t = 0; t < 4; ++t) w.p[j][t] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[j] + 1024u * t, kk * kTileBytes, 0);
      } else {
        load_run<QB>(rq, qoff[j], kk * kTileBytes, w.run[j]);
        w.sb[j] = __builtin_amdgcn_raw_buffer_load_b32(rsb, sboff[j], kk * 256u, 0);
      }
    }
  };

  f32x16_v acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // one K tile: the next tile's X (loaded one tile ago) into the other LDS buffer, the X loads of
  // the tile after that and the next tile's weight loads (into `nxt`) go out first, then this
  // tile's weights (in `cur`) are dequantised into operand registers and the MFMAs run. All loads
  // are unconditional (past the end they re-read the last tile, unused): a branch would make the
  // compiler's wait counting assume the other path's loads are still in flight. The scheduling
  // barrier keeps the compiler from sinking the loads behind the MFMAs, which would expose their
  // latency at the next tile's store.
  auto step = [&](int kt, const WSet& cur, WSet& nxt) {
    store_x((kt + 1) & 1);
    load_x(min(kt + 2, nkt - 1));
    load_w(min(kt + 1, nkt - 1), nxt);
    __builtin_amdgcn_sched_barrier(0);
    // per 16-k subtile T: its two weight operands are dequantised just before its MFMAs (so the
    // VALU work interleaves with the matrix pipe) and the X operands of subtile T + 1 are read from
    // LDS one subtile ahead (8k prefill 37.5 -> 37.1 ms, A/B on one box); the MFMA order, and so
    // every sum, is the same as dequantising the whole K tile first
    const f16_t* at = As[kt & 1];
    f16x8_v avc[MT], avn[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) avc[i] = *(const f16x8_v*)(at + (32 * i + c32) * LDSK + 32 * hf);
    f16x2_v s2[2], b2[2];
    if constexpr (!F16) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f16x2_v sbv = __builtin_bit_cast(f16x2_v, cur.sb[j]);
        s2[j] = __builtin_shufflevector(sbv, sbv, 0, 0);
        b2[j] = __builtin_shufflevector(sbv, sbv, 1, 1);
      }
    }
    auto sub = [&](auto tc) {
      constexpr int T = decltype(tc)::value;
      if constexpr (T < 3) {
#pragma unroll
        for (int i = 0; i < MT; ++i) avn[i] = *(const f16x8_v*)(at + (32 * i + c32) * LDSK + 32 * hf + 8 * (T + 1));
      }
      f16x8_v b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (F16) b[j] = __builtin_bit_cast(f16x8_v, cur.p[j][T]);
        else b[j] = deq8<QB, T>(cur.run[j], s2[j], b2[j]);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(avc[i], b[j], acc[i][j], 0, 0, 0);
      if constexpr (T < 3) {
#pragma unroll
        for (int i = 0; i < MT; ++i) avc[i] = avn[i];
      }
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    sub(std::integral_constant<int, 2>{});
    sub(std::integral_constant<int, 3>{});
    __syncthreads();
  };

  WSet w0, w1;
  load_x(kt0);
  load_w(kt0, w0);
  store_x(0);
  load_x(kt0 + 1);
  __syncthreads();
  for (int kt = kt0; kt < nkt; kt += 2) {   // kt0 and nkt are even
    step(kt, w0, w1);
    step(kt + 1, w1, w0);
  }

  // epilogue: acc[i][j][v] is X row m0 + 32i + 8(v/4) + 4(lane/32) + v%4 against row c32 of tile wtile[j]
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + 32 * i + 8 * (v >> 2) + 4 * hf + (v & 3);
      if (row >= M) continue;
      if constexpr (EPI == GEMM_SWIGLU) {
        const float g = acc[i][0][v], u = acc[i][1][v];
        a.y[(size_t)row * a.ldy + wrow0] = f2h_sep(g / (1.f + __expf(-g)) * u);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = blockIdx.y * BN + 64 * wave + 32 * j + c32;
          if (col < N) yout[(size_t)row * a.ldy + col] = acc[i][j][v];
        }
      }
    }
  }
}

size_t gemm_codes_bytes(int n, int k, int bits) { return (size_t)((n + 31) / 32) * (k / BK) * 256u * bits; }
size_t gemm_sb_bytes(int n, int k) { return (size_t)((n + 31) / 32) * (k / BK) * 256u; }
size_t gemm_w16_bytes(int n, int k) { return (size_t)((n + 31) / 32) * (k / BK) * 4096u; }

// One wave per (32-row, 64-k) tile: lane l dequantises its 32 codes with the GEMM's own deq8 and
// writes them as the four 16-byte planes of the fp16 copy.
template <int BITS>
__global__ void __launch_bounds__(64) k_repack16(GemmW w, uint32_t* w16, int nk) {
  const size_t tile = blockIdx.x;          // wtile * nk + kt
  const int lane = threadIdx.x;
  constexpr uint32_t kTileBytes = 256u * BITS;
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(w.codes, (uint32_t)w.ntile * nk * kTileBytes);
  Run<BITS> run;
  load_run<BITS>(rq, (uint32_t)lane * Planes<BITS>::PB, (uint32_t)(tile * kTileBytes), run);
  const f16x2_v sbv = __builtin_bit_cast(f16x2_v, w.sb[tile * 64 + lane]);
  const f16x2_v s2 = __builtin_shufflevector(sbv, sbv, 0, 0), b2 = __builtin_shufflevector(sbv, sbv, 1, 1);
  u32x4_v* out = (u32x4_v*)(w16 + tile * 1024);
  out[0 * 64 + lane] = __builtin_bit_cast(u32x4_v, deq8<BITS, 0>(run, s2, b2));
  out[1 * 64 + lane] = __builtin_bit_cast(u32x4_v, deq8<BITS, 1>(run, s2, b2));
  out[2 * 64 + lane] = __builtin_bit_cast(u32x4_v, deq8<BITS, 2>(run, s2, b2));
  out[3 * 64 + lane] = __builtin_bit_cast(u32x4_v, deq8<BITS, 3>(run, s2, b2));
}

hipError_t launch_repack_gemm16(hipStream_t s, const GemmW& w, uint32_t* w16) {
  if (!w.codes || !w.sb || !w16 || w.k % BK || w.ntile != (w.n + 31) / 32) return hipErrorInvalidValue;
  const int nk = w.k / BK;
  const size_t tiles = (size_t)w.ntile * nk;
  if (tiles == 0 || tiles > 0x7fffffff || tiles * 4096u > 0xffffffffull) return hipErrorInvalidValue;
  switch (w.bits) {
    case 4: hipLaunchKernelGGL(k_repack16<4>, dim3((unsigned)tiles), dim3(64), 0, s, w, w16, nk); break;
    case 6: hipLaunchKernelGGL(k_repack16<6>, dim3((unsigned)tiles), dim3(64), 0, s, w, w16, nk); break;
    case 8: hipLaunchKernelGGL(k_repack16<8>, dim3((unsigned)tiles), dim3(64), 0, s, w, w16, nk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The fp16 operand copy of a linear stored as bf16, NVFP4 or block-FP8: one wave per (32-row,
// 64-k) tile, lane l writes its four planes of f16(weight_value) (rows past N repeat row N - 1).
__global__ void __launch_bounds__(64) k_make_w16(QLinear w, uint32_t* w16, int nk) {
  const size_t tile = blockIdx.x;          // wtile * nk + kt
  const int lane = threadIdx.x;
  const int nt = (int)(tile / nk), kt = (int)(tile - (size_t)nt * nk);
  const int row = min(nt * 32 + (lane & 31), w.n - 1);
  const int k0 = kt * BK + 32 * (lane >> 5);
  u32x4_v* out = (u32x4_v*)(w16 + tile * 1024);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + 8 * t + 2 * i;
      p[i] = (uint32_t)f2h(weight_value(w, row, k)) | ((uint32_t)f2h(weight_value(w, row, k + 1)) << 16);
    }
    out[t * 64 + lane] = u32x4_v{p[0], p[1], p[2], p[3]};
  }
}

hipError_t launch_make_w16(hipStream_t s, const QLinear& w, uint32_t* w16) {
  if (w.fmt == FMT_AFFINE || !w16 || w.k % BK) return hipErrorInvalidValue;
  const int nk = w.k / BK;
  const size_t tiles = (size_t)((w.n + 31) / 32) * nk;
  if (tiles == 0 || tiles > 0x7fffffff || tiles * 4096u > 0xffffffffull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_make_w16, dim3((unsigned)tiles), dim3(64), 0, s, w, w16, nk);
  return hipGetLastError();
}

// One block of 64 threads per (32-row, 64-k) tile; thread l writes lane l's codes and (scale,
// bias) pair of the re-tiled copy (the layout is described with GemmW).
template <int BITS>
__global__ void __launch_bounds__(64) k_repack(QLinear w, uint8_t* codes, uint32_t* sb, int nk) {
  constexpr int PB = Planes<BITS>::PB, NP = Planes<BITS>::NP;
  const int blk = blockIdx.x, lane = threadIdx.x;
  const int nt = blk / nk, kt = blk - nt * nk;
  const int row = min(nt * 32 + (lane & 31), w.n - 1);
  const int k0 = kt * BK + 32 * (lane >> 5);
  const uint32_t* src = (const uint32_t*)(w.q + (size_t)row * ((size_t)w.k * BITS / 8) + (size_t)k0 * BITS / 8);
  uint32_t v[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) v[i] = src[i];
  if constexpr (BITS == 4) {
    // code j of each word to nibble 0, 2, 4, 6, 1, 3, 5, 7
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t o = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) o |= ((v[i] >> (4 * j)) & 0xFu) << (4 * (j < 4 ? 2 * j : 2 * (j - 4) + 1));
      v[i] = o;
    }
  }
  uint8_t* dst = codes + (size_t)blk * 256u * BITS + (size_t)lane * PB;
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int d = 0; d < PB / 4; ++d) ((uint32_t*)(dst + (size_t)p * 64 * PB))[d] = v[p * (PB / 4) + d];
  const int ngr = w.k / w.group;
  const int g = k0 / w.group;
  const f16_t s16 = f2h(bf2f(w.scales[(size_t)row * ngr + g])), b16 = f2h(bf2f(w.biases[(size_t)row * ngr + g]));
  sb[(size_t)blk * 64 + lane] = (uint32_t)s16 | ((uint32_t)b16 << 16);
}

hipError_t launch_repack_gemm(hipStream_t s, const QLinear& w, uint8_t* codes, uint32_t* sb) {
  if (w.k % (2 * BK) || w.group % 32 || (uintptr_t)codes % 16 || (uintptr_t)sb % 4) return hipErrorInvalidValue;
  const int nk = w.k / BK, nt = (w.n + 31) / 32;
  switch (w.bits) {
    case 4: hipLaunchKernelGGL(k_repack<4>, dim3(nt * nk), dim3(64), 0, s, w, codes, sb, nk); break;
    case 6: hipLaunchKernelGGL(k_repack<6>, dim3(nt * nk), dim3(64), 0, s, w, codes, sb, nk); break;
    case 8: hipLaunchKernelGGL(k_repack<8>, dim3(nt * nk), dim3(64), 0, s, w, codes, sb, nk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS, int BMT>
static void launch_bm(hipStream_t s, const GemmArgs& a) {
  const int gm = (a.m + BMT - 1) / BMT;
  if (a.epi == GEMM_SWIGLU) {
    hipLaunchKernelGGL((k_gemm<BITS, GEMM_SWIGLU, BMT>), dim3(gm, a.w.n / BN), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_gemm<BITS, GEMM_STORE, BMT>), dim3(gm, (a.w.n + BN - 1) / BN, a.yf2 ? 2 : 1), dim3(256), 0, s, a);
  }
}

template <int BITS>
static hipError_t launch_bits(hipStream_t s, const GemmArgs& a) {
  // 128-row tiles (each weight code is loaded once per 128 rows of X) from 2048 weight rows up
  // (the hidden-width outputs fill the chip through their K split; 64-row tiles there measured 1%
  // slower over the 8k prefill); 64-row tiles for narrower ones, which would leave most CUs idle
  if (a.w.n >= 2048) launch_bm<BITS, 128>(s, a);
  else launch_bm<BITS, 64>(s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(hipStream_t s, const GemmArgs& a) {
  if (a.m <= 0) return hipSuccess;
  // 16-byte rows of X, an even number of K tiles, 32-code runs inside one group, whole SwiGLU tiles
  if (a.w.k % (2 * BK) || (!a.w.w16 && a.w.group % 32) || a.ldx % 8 || (uintptr_t)a.x % 16 || (uintptr_t)a.x_lo % 16 ||
      a.w.ntile != (a.w.n + 31) / 32 || (a.epi == GEMM_SWIGLU && a.w.n % BN))
    return hipErrorInvalidValue;
  // a K split: two halves of an even number of K tiles, plain STORE
  if (a.yf2 && ((a.w.k / BK) % 4 || a.x_lo || a.epi != GEMM_STORE)) return hipErrorInvalidValue;
  if (a.w.w16) {
    if ((size_t)a.w.ntile * (a.w.k / BK) * 4096u > 0xffffffffull) return hipErrorInvalidValue;
    return launch_bits<16>(s, a);
  }
  switch (a.w.bits) {
    case 4: return launch_bits<4>(s, a);
    case 6: return launch_bits<6>(s, a);
    case 8: return launch_bits<8>(s, a);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------------------------
// Decode linears at 3 .. 64 operand rows ("skinny" MFMA GEMM). One block per 32-row weight tile
// (SwiGLU: the gate tile and its up tile); the four waves take every fourth K tile (with the loads
// of the next 2-4 of them in flight), each accumulating MT x NT MFMA tiles over all input rows
// (x rows, then the x_lo rows when the input is carried as a pair), with the weights dequantised
// straight into operand registers from the re-tiled copy and the input rows read from L2 in
// contiguous row segments and staged through a per-wave LDS slice (loading each lane's own operand
// rows straight from L2 touched 64 row segments per load: 7.19k -> 7.41k tok/s at 8 streams). The
// four partial tiles meet in LDS and are added in wave order; the epilogue (the GEMV's) runs one
// thread per (row, column): the pair's two rows are added (x row first), then STORE, SwiGLU, or
// the head's logits with each row's argmax key. The conv layers' in_proj runs here as a plain
// STORE over all 192 tiles; the gated conv follows in its own launch (k_conv, decode mode).
// ---------------------------------------------------------------------------------------------

template <int EPI> struct SgTiles { static constexpr int v = EPI == GEMV_SWIGLU ? 2 : 1; };
// Whether the waves' partial tiles exceed 96 KB of LDS together (then they are reduced per column tile).
template <int EPI, int MT, int WV> struct SgTwoPhase {
  static constexpr bool v = (size_t)WV * MT * 32 * SgTiles<EPI>::v * 32 * sizeof(float) > 96 * 1024;
};
constexpr int kHeadTiles = 4;    // 32-row tiles of the head per block

// STORE with g.yf_part set: blockIdx.y = K quarter (the block's waves share that quarter's tiles).
template <int BITS, int EPI, int MT, int WV>
__global__ void __launch_bounds__(64 * WV) k_sgemm(GemmW w, GemvArgs g) {
  constexpr bool F16 = BITS == 16;             // operands from the fp16 copy (GemmW::w16)
  constexpr int QB = F16 ? 4 : BITS;
  constexpr int NT = SgTiles<EPI>::v;
  constexpr int NTH = 64 * WV;
  static_assert(EPI != GEMV_LOGITS || WV == 4, "the head's argmax slots assume 256 threads");
  constexpr int D = MT == 1 ? 4 : 2;   // K tiles in flight per wave
  constexpr int TW = NT * 32, TR = MT * 32;
  constexpr uint32_t kTileBytes = F16 ? 4096u : 256u * BITS;
  extern __shared__ __attribute__((aligned(16))) float sg_smem[];   // [WV][TR][32] partials, [TR][TW] sums
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, c32 = lane & 31;
  const int R = g.batch;
  const bool pair = g.x_lo != nullptr;
  const int Meff = pair ? 2 * R : R;
  const int N = w.n, K = w.k;
  const int nk = K / BK;

  // the head: each block takes kHeadTiles consecutive 32-row tiles and keeps every row's best key
  // across them, so the rows' argmax keys take one partial store per block (not per tile)
  constexpr int TPB = EPI == GEMV_LOGITS ? kHeadTiles : 1;
  uint64_t best[8] = {0, 0, 0, 0, 0, 0, 0, 0};   // per epilogue slot idx = tid + 256 k (rows < 64)
  for (int tt = 0; tt < TPB; ++tt) {
  const int tb = blockIdx.x * TPB + tt;
  if (EPI == GEMV_LOGITS && tb >= w.ntile) break;
  int tile[NT];
  if constexpr (EPI == GEMV_SWIGLU) {
    tile[0] = tb;
    tile[1] = (N / 2) / 32 + tb;
  } else {
    tile[0] = tb;
  }
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(F16 ? (const void*)w.w16 : (const void*)w.codes, (uint32_t)w.ntile * nk * kTileBytes);
  const __amdgpu_buffer_rsrc_t rsb = rsrc_of(F16 ? (const void*)w.w16 : (const void*)w.sb, (uint32_t)w.ntile * nk * 256u);
  uint32_t qoff[NT], sboff[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    qoff[j] = (uint32_t)tile[j] * nk * kTileBytes + (uint32_t)lane * (F16 ? 16u : (uint32_t)Planes<QB>::PB);
    sboff[j] = ((uint32_t)tile[j] * nk * 64u + lane) * 4u;
  }
  // input rows of a K tile: piece q holds virtual rows 8q .. 8q + 7 (x rows, then x_lo rows), lane
  // l row 8q + l / 8, 16-byte chunk l % 8 (contiguous 128-byte row segments); only pieces with a
  // real row are loaded. Each wave stages its tile's rows in its own LDS slice (rows of kXld
  // halves) and reads the MFMA A operands from there; rows past Meff hold anything (their MFMA
  // rows are never read).
  constexpr int kXld = 72;
  f16_t* const xslice = (f16_t*)sg_smem + (size_t)wave * (32 * MT * kXld);
  const f16_t* xrow[4 * MT];
#pragma unroll
  for (int q = 0; q < 4 * MT; ++q) {
    const int vr = 8 * q + (lane >> 3);
    xrow[q] = (vr < R ? g.x + (size_t)vr * g.ldx : vr < Meff ? g.x_lo + (size_t)(vr - R) * g.ldx : g.x) + 8 * (lane & 7);
  }

  struct WSet {
    Run<QB> run[F16 ? 1 : NT];
    uint32_t sb[F16 ? 1 : NT];
    u32x4_v p[F16 ? NT : 1][F16 ? 4 : 1];   // fp16 copy: the operand registers themselves
    u32x4_v xr[4 * MT];
  };
  // K tiles [k0, k0 + nkb) of this block; this wave's: k0 + wave, k0 + wave + WV, ...
  const int nkb = nk / gridDim.y, k0 = blockIdx.y * nkb;
  const int ns = (nkb - wave + WV - 1) / WV;
  auto load = [&](int s, WSet& ws) {
    const int kt = k0 + wave + WV * min(s, ns - 1);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (F16) {
#pragma unroll
        for (int t = 0; t < 4; ++t) ws.p[j][t] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[j] + 1024u * t, (uint32_t)kt * kTileBytes, 0);
      } else {
        load_run<QB>(rq, qoff[j], (uint32_t)kt * kTileBytes, ws.run[j]);
        ws.sb[j] = __builtin_amdgcn_raw_buffer_load_b32(rsb, sboff[j], (uint32_t)kt * 256u, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < 4 * MT; ++q)
      if (8 * q < Meff) ws.xr[q] = *(const u32x4_v*)(xrow[q] + kt * BK);
  };
  f32x16_v acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto compute = [&](const WSet& ws) {
#pragma unroll
    for (int q = 0; q < 4 * MT; ++q)
      if (8 * q < Meff) *(u32x4_v*)(xslice + (8 * q + (lane >> 3)) * kXld + 8 * (lane & 7)) = ws.xr[q];
    u32x4_v av[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) av[i][t] = *(const u32x4_v*)(xslice + (32 * i + c32) * kXld + 32 * hf + 8 * t);
    f16x2_v s2[NT], b2[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const f16x2_v sbv = __builtin_bit_cast(f16x2_v, ws.sb[F16 ? 0 : j]);
      s2[j] = __builtin_shufflevector(sbv, sbv, 0, 0);
      b2[j] = __builtin_shufflevector(sbv, sbv, 1, 1);
    }
    auto sub = [&](auto tc) {
      constexpr int T = decltype(tc)::value;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        f16x8_v b;
        if constexpr (F16) b = __builtin_bit_cast(f16x8_v, ws.p[j][T]);
        else b = deq8<QB, T>(ws.run[F16 ? 0 : j], s2[j], b2[j]);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_v, av[i][T]), b, acc[i][j], 0, 0, 0);
      }
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    sub(std::integral_constant<int, 2>{});
    sub(std::integral_constant<int, 3>{});
  };
  // D register sets in a ring: the loads of the wave's next D K tiles are in flight while one is
  // computed (the K loop of a decode linear is latency-bound: few tiles per wave, one block per
  // CU). Branch-free: past the end the loads re-read the wave's last tile and are not computed.
  WSet ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, ring[d]);
  for (int s = 0; s < ns; s += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (s + d < ns) compute(ring[d]);
      load(s + d + D, ring[d]);
    }
  }

  __syncthreads();   // every wave is done with its input slice (the partials reuse that LDS)
  // the partial tiles: acc[i][j][v] is virtual row 32i + 8(v/4) + 4(lane/32) + v%4, column
  // 32j + lane%32 of the block's tile; an element's total adds the waves' partials in wave order.
  // All waves' tiles at once when they fit (SgTwoPhase false), else one column tile at a time
  // into a table of sums (the same additions in the same order).
  auto total = [&](int vr, int col) {
    if constexpr (SgTwoPhase<EPI, MT, WV>::v) {
      return sg_smem[WV * TR * 32 + vr * TW + col];
    } else {
      const int e = vr * TW + col;
      float t = sg_smem[e];
#pragma unroll
      for (int q = 1; q < WV; ++q) t += sg_smem[q * TR * TW + e];
      return t;
    }
  };
  if constexpr (SgTwoPhase<EPI, MT, WV>::v) {
    float* part = sg_smem;
    float* sums = sg_smem + WV * TR * 32;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float* mine = part + (size_t)wave * TR * 32;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) mine[(32 * i + 8 * (v >> 2) + 4 * hf + (v & 3)) * 32 + c32] = acc[i][j][v];
      __syncthreads();
      for (int e = tid; e < TR * 32; e += NTH) {
        float t = part[e];
#pragma unroll
        for (int q = 1; q < WV; ++q) t += part[q * TR * 32 + e];
        sums[(e >> 5) * TW + 32 * j + (e & 31)] = t;
      }
      __syncthreads();
    }
  } else {
    float* mine = sg_smem + (size_t)wave * TR * TW;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) mine[(32 * i + 8 * (v >> 2) + 4 * hf + (v & 3)) * TW + 32 * j + c32] = acc[i][j][v];
    __syncthreads();
  }
  auto val = [&](int r, int col) {
    float v = total(r, col);
    if (pair) v = v + total(r + R, col);
    return v;
  };
  for (int idx = tid; idx < R * 32; idx += NTH) {
    const int r = idx >> 5, c = idx & 31;
    if constexpr (EPI == GEMV_LOGITS) {
      // logits, and the running argmax key of the row (order key, then the lower id)
      const int n = 32 * tile[0] + c;
      const float v = val(r, c);
      if (n < N) {
        if (g.logits) g.logits[(size_t)r * g.ld_logits + n] = v;
        const uint64_t key = ((uint64_t)order_key(v) << 32) | (uint64_t)(0xffffffffu - (uint32_t)n);
        best[idx >> 8] = key > best[idx >> 8] ? key : best[idx >> 8];
      }
    } else if constexpr (EPI == GEMV_STORE) {
      const int n = 32 * tile[0] + c;
      float* out = blockIdx.y == 0 ? g.yf : g.yf_part[blockIdx.y - 1];
      if (n < N) out[(size_t)r * g.ldy + n] = val(r, c);
    } else {
      static_assert(EPI == GEMV_SWIGLU, "STORE, SwiGLU or the head");
      const float gt = val(r, c), up = val(r, 32 + c);
      g.y[(size_t)r * g.ldy + 32 * tb + c] = f2h_sep(gt / (1.f + __expf(-gt)) * up);
    }
  }
  __syncthreads();   // the LDS tiles are reused by the next tile
  }
  if constexpr (EPI == GEMV_LOGITS) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (tid + 256 * k >= R * 32) break;
      uint64_t key = best[k];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)key, o, 64), hi = __shfl_xor((uint32_t)(key >> 32), o, 64);
        const uint64_t other = ((uint64_t)hi << 32) | lo;
        key = other > key ? other : key;
      }
      if ((tid & 31) == 0) g.keys[(size_t)((tid + 256 * k) >> 5) * kArgmaxParts + blockIdx.x] = key;
    }
  }
}

template <int BITS, int EPI, int MT, int WV>
static hipError_t launch_sg(hipStream_t s, const GemmW& w, const GemvArgs& g, int blocks, int ksplit) {
  const size_t part = SgTwoPhase<EPI, MT, WV>::v ? ((size_t)WV * MT * 32 * 32 + (size_t)MT * 32 * SgTiles<EPI>::v * 32) * sizeof(float)
                                                 : (size_t)WV * MT * 32 * SgTiles<EPI>::v * 32 * sizeof(float);
  const size_t xs = (size_t)WV * 32 * MT * 72 * sizeof(f16_t);
  const size_t lds = part > xs ? part : xs;
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_sgemm<BITS, EPI, MT, WV>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_sgemm<BITS, EPI, MT, WV>), dim3(blocks, ksplit), dim3(64 * WV), lds, s, w, g);
  return hipGetLastError();
}

// Four waves per block (eight for the longer 4-bit plain linears), each needing at least one K
// tile of the block's range. The wave count depends on the weight format and shape alone, never on
// the row count, so a row's sums do not depend on its batch.
template <int BITS, int EPI>
static hipError_t launch_sg_epi(hipStream_t s, const GemmW& w, const GemvArgs& g, int blocks, int meff, int ksplit = 1) {
  const int nkb = (w.k / BK) / ksplit;
  if (nkb < 4) return hipErrorInvalidValue;
  if constexpr (EPI == GEMV_STORE && BITS == 4) {
    // 4-bit plain linears with at least 16 K tiles a block (w2's K quarters, qkvg, in_proj): 8 waves,
    // each walking half as many K tiles (8 streams 7,657 -> 7,782 tok/s; at 8 bits and from the fp16
    // copy the same lost 1.4% and 4.6%, and with the 8-tile K quarters of the 2048-wide
    // projections as well it gained less)
    if (nkb >= 16)
      return meff <= 32 ? launch_sg<BITS, EPI, 1, 8>(s, w, g, blocks, ksplit) : launch_sg<BITS, EPI, 2, 8>(s, w, g, blocks, ksplit);
  }
  return meff <= 32 ? launch_sg<BITS, EPI, 1, 4>(s, w, g, blocks, ksplit) : launch_sg<BITS, EPI, 2, 4>(s, w, g, blocks, ksplit);
}

template <int BITS>
static hipError_t launch_sg_bits(hipStream_t s, const GemmW& w, const GemvArgs& g, int meff) {
  switch (g.epi) {
    case GEMV_STORE: {
      // narrow outputs (fewer than 128 tiles: one block per tile would leave most CUs idle) split
      // K in four quarters when the caller provides the partial outputs
      const bool ks = g.yf_part[0] && g.yf_part[1] && g.yf_part[2] && sgemm_store_ksplit(w);
      return launch_sg_epi<BITS, GEMV_STORE>(s, w, g, w.ntile, meff, ks ? 4 : 1);
    }
    case GEMV_SWIGLU: return launch_sg_epi<BITS, GEMV_SWIGLU>(s, w, g, w.n / 64, meff);
    case GEMV_LOGITS:
      if ((w.ntile + kHeadTiles - 1) / kHeadTiles > kArgmaxParts) return hipErrorInvalidValue;
      return launch_sg_epi<BITS, GEMV_LOGITS>(s, w, g, (w.ntile + kHeadTiles - 1) / kHeadTiles, meff);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sgemm(hipStream_t s, const GemmW& w, const GemvArgs& g) {
  const int meff = g.x_lo ? 2 * g.batch : g.batch;
  if (g.batch < 1 || meff > 64 || w.k % (4 * BK) || (w.codes && w.group % 32) || g.ldx % 8 || (uintptr_t)g.x % 16 ||
      (uintptr_t)g.x_lo % 16 || w.ntile != (w.n + 31) / 32 ||
      (g.epi == GEMV_SWIGLU && w.n % 64) || g.epi == GEMV_CONV)
    return hipErrorInvalidValue;
  // the fp16 copy only where there are no codes (bf16, NVFP4, block-FP8): decode reads the fewest
  // bytes from the codes
  if (!w.codes) {
    if (!w.w16 || (size_t)w.ntile * (w.k / BK) * 4096u > 0xffffffffull) return hipErrorInvalidValue;
    return launch_sg_bits<16>(s, w, g, meff);
  }
  switch (w.bits) {
    case 4: return launch_sg_bits<4>(s, w, g, meff);
    case 6: return launch_sg_bits<6>(s, w, g, meff);
    case 8: return launch_sg_bits<8>(s, w, g, meff);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lfm3
