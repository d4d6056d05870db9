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

// Rows handled together by one wave: 8 for STORE / LOGITS, 4 gate + the 4 matching up rows for
// SWIGLU, B, C and x rows of 2 channels (6) for the conv epilogue.
template <int EPI> struct RowsPerGroup { static constexpr int v = EPI == GEMV_CONV ? 6 : 8; };

template <int EPI> LFM3_HOST_DEV int n_groups_of(int N) {
  if (EPI == GEMV_SWIGLU) return N / 8;
  if (EPI == GEMV_CONV) return N / 6;
  return (N + 7) / 8;
}

template <int EPI> LFM3_DEV void rows_of(int g, int N, int (&rows)[RowsPerGroup<EPI>::v]) {
  if constexpr (EPI == GEMV_SWIGLU) {
    const int half = N / 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) { rows[r] = 4 * g + r; rows[4 + r] = half + 4 * g + r; }
  } else if constexpr (EPI == GEMV_CONV) {
    const int third = N / 3;
#pragma unroll
    for (int j = 0; j < 3; ++j) { rows[2 * j] = j * third + 2 * g; rows[2 * j + 1] = j * third + 2 * g + 1; }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) rows[r] = min(8 * g + r, N - 1);
  }
}

// Stage the fp16 input rows in LDS in chunk pair order, with per-chunk sums of the staged values.
// Either x comes from global fp16 rows (PRO = 0), or (PRO = 1) the decode norm prologue forms it:
// h_new = h_src + rmsnorm(m) * w_post (or h_src), x = f16(rmsnorm(h_new) * w_pre); block 0 also
// stores h_new, the capture rows and the fp32 x. The arithmetic matches k_resid_norm exactly.
constexpr int kP = 16;  // prologue elements per thread: K = hidden <= 4096

template <int BT> struct PrologueRegs {
  float hv[BT][kP], mv[BT][kP], wpo[kP], wpr[kP];
};

// All prologue loads, unconditional (absent inputs read a valid stand-in and are masked later),
// so they are issued back to back before the weight prefetch.
template <int BT>
LFM3_DEV void prologue_load(const GemvArgs& a, PrologueRegs<BT>& p) {
  const int K = a.w.k, tid = threadIdx.x;
  const float* mp = a.m ? a.m : a.h_src;
  const bf16_t* wpo = a.w_post ? a.w_post : a.w_pre;
#pragma unroll
  for (int i = 0; i < kP; ++i) {
    const int k = min(tid + 256 * i, K - 1);
    p.wpr[i] = bf2f(a.w_pre[k]);
    p.wpo[i] = bf2f(wpo[k]);
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const size_t o = (size_t)min(b, a.batch - 1) * K + k;
      p.hv[b][i] = a.h_src[o];
      p.mv[b][i] = mp[o];
    }
  }
}

template <int BITS>
LFM3_DEV void put_x(uint16_t* xp, float* xsum, int K, int b, int k, float x) {
  using Q = QT<BITS>;
  const int lane = threadIdx.x & 63;
  const int c = k / Q::CH, kk = k - c * Q::CH;
  xp[b * K + c * Q::CH + pair_pos<BITS>(kk)] = f2h(x);
  // element k = tid + 256 i: chunks of CH consecutive k sit in CH consecutive lanes of one wave
  float s16 = row16_sum(x);
  if (Q::CH == 32) s16 += __shfl_xor(s16, 16, 64);
  if ((lane & (Q::CH - 1)) == 0) xsum[b * (K / Q::CH) + c] = s16;
}

template <int BITS, int BT>
LFM3_DEV void prologue_compute(const GemvArgs& a, PrologueRegs<BT>& p, uint16_t* xp, float* xsum, float* red) {
  const int K = a.w.k;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int per = K / 256;
  if (a.m) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < kP; ++i)
        if (i < per) ss = fmaf(p.mv[b][i], p.mv[b][i], ss);
      ss = wave_sum(ss);
      if (lane == 0) red[wave * BT + b] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const float rm = rsqrtf((red[b] + red[BT + b] + red[2 * BT + b] + red[3 * BT + b]) / (float)K + a.eps);
#pragma unroll
      for (int i = 0; i < kP; ++i) p.hv[b][i] = fmaf(p.mv[b][i] * rm, p.wpo[i], p.hv[b][i]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kP; ++i)
      if (i < per) ss = fmaf(p.hv[b][i], p.hv[b][i], ss);
    ss = wave_sum(ss);
    if (lane == 0) red[wave * BT + b] = ss;
  }
  __syncthreads();
  const bool first = blockIdx.x == 0;
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const float rh = rsqrtf((red[b] + red[BT + b] + red[2 * BT + b] + red[3 * BT + b]) / (float)K + a.eps);
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      if (i < per) {
        const int k = tid + 256 * i;
        const float x = (p.hv[b][i] * rh) * p.wpr[i];
        put_x<BITS>(xp, xsum, K, b, k, b < a.batch ? h2f(f2h_sep(x)) : 0.f);
        if (first && b < a.batch) {
          if (a.m && a.h_dst) a.h_dst[(size_t)b * K + k] = p.hv[b][i];
          if (a.capture) a.capture[(size_t)b * a.capture_ld + k] = p.hv[b][i];
          if (a.x_copy) a.x_copy[(size_t)b * K + k] = x;
        }
      }
    }
  }
}

template <int BITS, int BT>
LFM3_DEV void stage_plain(const GemvArgs& a, uint16_t* xp, float* xsum) {
  const int K = a.w.k, tid = threadIdx.x;
  const int per = K / 256;
  for (int i0 = 0; i0 < per; i0 += kP) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      uint16_t xr[kP];
      const f16_t* row = a.x + (size_t)min(b, a.batch - 1) * a.ldx;
#pragma unroll
      for (int i = 0; i < kP; ++i) xr[i] = row[min(tid + 256 * (i0 + i), K - 1)];
#pragma unroll
      for (int i = 0; i < kP; ++i)
        if (i0 + i < per) put_x<BITS>(xp, xsum, K, b, tid + 256 * (i0 + i), b < a.batch ? h2f(xr[i]) : 0.f);
    }
  }
}

template <int BITS, int BT, int EPI, int PRO>
__global__ void __launch_bounds__(256) k_gemv(GemvArgs a) {
  using Q = QT<BITS>;
  constexpr int RG = RowsPerGroup<EPI>::v;
  extern __shared__ uint32_t smem[];
  __shared__ float red[4 * BT];
  const int K = a.w.k;
  const int NC = K / Q::CH;
  const int NIT = (NC + 63) / 64;
  uint16_t* xp = (uint16_t*)smem;                 // [BT][K] fp16 in pair order
  float* xsum = (float*)(smem + (BT * K) / 2);    // [BT][NC]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = a.w.n;
  const int n_groups = n_groups_of<EPI>(N);
  const size_t row_bytes = (size_t)K * BITS / 8;
  const int ngr = K / a.w.group;
  const int gstride = gridDim.x * 4;

  // The wave walks a flat sequence of (group, chunk) steps. Weights for step s + 1 are loaded
  // into the other of two register sets while step s is computed (no copies between them, so no
  // wait beyond the one the compute needs). Loads are branch-free: out-of-range steps load a valid
  // clamped address and are not computed.
  struct WRegs {
    uint32_t q[RG][Q::NDW];
    bf16_t s[RG], b[RG];   // raw bits: converted when used
  };
  const int g0 = blockIdx.x * 4 + wave;
  const int nsteps = g0 < n_groups ? ((n_groups - 1 - g0) / gstride + 1) * NIT : 0;
  auto fetch = [&](WRegs& W, int step) {
    const int gi = step / NIT, it = step - gi * NIT;
    const int c = min(lane + 64 * it, NC - 1);
    int rows[RG];
    rows_of<EPI>(min(g0 + gi * gstride, n_groups - 1), N, rows);
    const int grp = (c * Q::CH) / a.w.group;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const uint32_t* src = (const uint32_t*)(a.w.q + (size_t)rows[r] * row_bytes + (size_t)c * (Q::CH * BITS / 8));
      if constexpr (Q::NDW == 4) {
        const u32x4_v v = __builtin_nontemporal_load((const u32x4_v*)src);
        W.q[r][0] = v[0]; W.q[r][1] = v[1]; W.q[r][2] = v[2]; W.q[r][3] = v[3];
      } else {
#pragma unroll
        for (int d = 0; d < Q::NDW; ++d) W.q[r][d] = __builtin_nontemporal_load(src + d);
      }
      W.s[r] = a.w.scales[(size_t)rows[r] * ngr + grp];
      W.b[r] = a.w.biases[(size_t)rows[r] * ngr + grp];
    }
  };

  WRegs wa, wb;
  if constexpr (PRO) {
    // prologue loads first, then the weight prefetch, then the prologue arithmetic: the in-order
    // load counter then lets the weights stay in flight through the prologue
    PrologueRegs<BT> p;
    prologue_load<BT>(a, p);
    __builtin_amdgcn_sched_barrier(0);
    fetch(wa, 0);
    __builtin_amdgcn_sched_barrier(0);
    prologue_compute<BITS, BT>(a, p, xp, xsum, red);
  } else {
    stage_plain<BITS, BT>(a, xp, xsum);
    fetch(wa, 0);
  }
  __syncthreads();

  uint64_t best[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) best[b] = 0;
  float acc[RG][BT];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;

  auto consume = [&](const WRegs& W, int step) {
    const int gi = step / NIT, it = step - gi * NIT;
    const int c = lane + 64 * it;
    if (c < NC) {
      uint32_t xv[BT][Q::NP];
      float X[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const uint4* xs4 = (const uint4*)(xp + b * K + c * Q::CH);
#pragma unroll
        for (int q = 0; q < Q::NP / 4; ++q) {
          const uint4 v = xs4[q];
          xv[b][4 * q] = v.x; xv[b][4 * q + 1] = v.y; xv[b][4 * q + 2] = v.z; xv[b][4 * q + 3] = v.w;
        }
        X[b] = xsum[b * NC + c];
      }
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        uint32_t wp[Q::NP];
        unpack<BITS>(W.q[r], wp);
        const float sc = bf2f(W.s[r]), bi = bf2f(W.b[r]);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          float d = 0.f;
#pragma unroll
          for (int p = 0; p < Q::NP; ++p) d = dot2(wp[p], xv[b][p], d);
          acc[r][b] += fmaf(sc, d - kMagicOff * X[b], bi * X[b]);
        }
      }
    }
    if (it != NIT - 1) return;
    const int g = g0 + gi * gstride;
    // totals are wave-uniform after wave_sum
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = wave_sum(acc[r][b]);
    if (lane == 0) {
      if constexpr (EPI == GEMV_STORE) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int b = 0; b < BT; ++b)
            if (b < a.batch && 8 * g + r < N) a.yf[(size_t)b * a.ldy + 8 * g + r] = acc[r][b];
      } else if constexpr (EPI == GEMV_SWIGLU) {
        // silu(a) * b is rounded to fp32, then to fp16, in every batch-size instance, so a row's
        // result does not depend on the batch it is decoded in
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            if (b >= a.batch) continue;
            const float gt = acc[j][b], up = acc[4 + j][b];
            const float sv = gt / (1.f + __expf(-gt)) * up;
            a.y[(size_t)b * a.ldy + 4 * g + j] = f2h_sep(sv);
          }
      } else if constexpr (EPI == GEMV_CONV) {
        // gated short conv of channels 2g, 2g+1 ("LFM3-1.7B port" table row 1): z = f16(B * x),
        // y = sum_j ker[c, j] * [state | z]_j, out = f16(C * y), state <- last taps-1 z
        const int H = N / 3, T = a.conv_taps, S = T - 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ch = 2 * g + j;
          float ker[kMaxTaps];
          for (int t = 0; t < T; ++t) ker[t] = bf2f(a.conv_kernel[(size_t)ch * T + t]);
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            if (b >= a.batch) continue;
            f16_t* st = a.conv_state + (size_t)a.conv_slot[b] * a.conv_slot_stride;
            const float z = h2f(f2h_sep(acc[j][b] * acc[4 + j][b]));
            float win[kMaxTaps];
            for (int t = 0; t < S; ++t) win[t] = h2f(st[(size_t)t * H + ch]);
            float y = ker[S] * z;
            for (int t = 0; t < S; ++t) y = fmaf(ker[t], win[t], y);
            for (int t = 0; t + 1 < S; ++t) st[(size_t)t * H + ch] = f2h(win[t + 1]);
            st[(size_t)(S - 1) * H + ch] = f2h(z);
            a.y[(size_t)b * a.ldy + ch] = f2h_sep(acc[2 + j][b] * y);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int n = 8 * g + r;
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
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;
  };

  for (int step = 0; step < nsteps; step += 2) {
    fetch(wb, step + 1);
    consume(wa, step);
    fetch(wa, step + 2);
    if (step + 1 < nsteps) consume(wb, step + 1);
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
  const int n_groups = a.epi == GEMV_SWIGLU ? n_groups_of<GEMV_SWIGLU>(N)
                       : a.epi == GEMV_CONV ? n_groups_of<GEMV_CONV>(N) : n_groups_of<GEMV_STORE>(N);
  int grid = (n_groups + 3) / 4;
  const int cap = a.max_blocks > 0 ? a.max_blocks : 1024;
  if (grid > cap) grid = cap;
  if (a.h_src) {
    if constexpr (BT <= 2) {
      switch (a.epi) {
        case GEMV_STORE: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE, 1>), dim3(grid), dim3(256), lds, s, a); break;
        case GEMV_SWIGLU: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_SWIGLU, 1>), dim3(grid), dim3(256), lds, s, a); break;
        case GEMV_CONV: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_CONV, 1>), dim3(grid), dim3(256), lds, s, a); break;
        default: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_LOGITS, 1>), dim3(grid), dim3(256), lds, s, a); break;
      }
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    switch (a.epi) {
      case GEMV_STORE: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE, 0>), dim3(grid), dim3(256), lds, s, a); break;
      case GEMV_SWIGLU: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_SWIGLU, 0>), dim3(grid), dim3(256), lds, s, a); break;
      case GEMV_CONV: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_CONV, 0>), dim3(grid), dim3(256), lds, s, a); break;
      default: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_LOGITS, 0>), dim3(grid), dim3(256), lds, s, a); break;
    }
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
    // split the batch into launches of at most bt rows (plain x input only)
    if (a.h_src) return hipErrorInvalidValue;
    for (int b0 = 0; b0 < a.batch; b0 += bt) {
      GemvArgs p = a;
      p.batch = a.batch - b0 < bt ? a.batch - b0 : bt;
      p.x = a.x + (size_t)b0 * a.ldx;
      for (int i = 0; i < p.batch; ++i) p.conv_slot[i] = a.conv_slot[b0 + i];
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
