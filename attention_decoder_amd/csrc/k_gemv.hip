// Fused dequant-GEMV for decode (batch 1..8) on gfx950.
//
// y[b, n] = sum_k x[b, k] * (q[n, k] * s[n, g] + bias[n, g]) with MLX affine weights (TensorFold
// issue #1491, "Checkpoint handling"). The weights are never rounded: per lane chunk of one group,
//   sum_k x_k (q_k s + bias) = s * sum_k x_k q_k + bias * sum_k x_k,
// where q_k enters an fp16 dot2 exactly as 1024 + q (exponent 2^10 with q in the 10-bit mantissa,
// built by one and-or per pair) and s * 1024 * sum x is subtracted. At 4 bits the odd nibbles of
// a byte are not shifted down: masked in place they read as 1024 + 16 q, also exact, and go to a
// second accumulator that is scaled by 1/16 (exact), so a code word costs one shift and four
// and-ors. x is fp16; accumulation is fp32.
//
// Layout: a wave owns a group of 4 rows (SwiGLU: 2 gate rows + the 2 matching up rows); lane l
// streams chunks l, l+64, ... of each row (16 B of codes: 32 4-bit or 16 8-bit codes; 12 B of
// 6-bit codes) and the chunk's scale/bias; x is staged once per block in LDS in the pair order the
// unpacked codes come in, with per-chunk sums of x.
#include "kernels.h"
#include "norm_vec.h"

namespace lfm3 {

// Chunk geometry of a weight format: CH weights per lane chunk, NDW dwords of codes, NP fp16 pairs
// after unpacking, CB code bits. BITS 4 / 6 / 8 are MLX affine codes; 16 stored bf16 weights; 41
// NVFP4 (e2m1 codes, an e4m3 scale per 16 k, an fp32 tensor scale); 48 block-FP8 (e4m3 codes, an
// fp32 scale per 128 x 128 block).
template <int BITS> struct QT;
template <> struct QT<4> { static constexpr int CH = 32, NDW = 4, NP = 16, CB = 4; };
template <> struct QT<6> { static constexpr int CH = 16, NDW = 3, NP = 8, CB = 6; };
template <> struct QT<8> { static constexpr int CH = 16, NDW = 4, NP = 8, CB = 8; };
template <> struct QT<16> { static constexpr int CH = 8, NDW = 4, NP = 4, CB = 16; };
template <> struct QT<41> { static constexpr int CH = 32, NDW = 4, NP = 16, CB = 4; };
template <> struct QT<48> { static constexpr int CH = 16, NDW = 4, NP = 8, CB = 8; };
// The pair order of a format's unpacked codes (NVFP4 pairs like 4-bit codes, block-FP8 like 8-bit).
template <int BITS> struct PairOrder { static constexpr int v = BITS == 41 ? 4 : BITS == 48 ? 8 : BITS; };
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

// Codes of one chunk as fp16 pairs. `magic` is kMagic2 held in a VGPR, so that each pair is one
// v_and_or_b32 (mask from an SGPR). 4-bit: pair 4d + j holds nibbles j and j + 4 of word d, as
// 1024 + q for even j and as 1024 + 16 q (nibble left at bits 4..7) for odd j.
template <int BITS> LFM3_DEV void unpack(const uint32_t (&w)[QT<BITS>::NDW], uint32_t (&p)[QT<BITS>::NP], uint32_t magic) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t w8 = w[d] >> 8;
      p[4 * d] = (w[d] & 0x000F000Fu) | magic;
      p[4 * d + 1] = (w[d] & 0x00F000F0u) | magic;
      p[4 * d + 2] = (w8 & 0x000F000Fu) | magic;
      p[4 * d + 3] = (w8 & 0x00F000F0u) | magic;
    }
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
      p[i] = (c[0] | (c[1] << 16)) | magic;
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      p[2 * d] = (w[d] & 0x00FF00FFu) | magic;
      p[2 * d + 1] = ((w[d] >> 8) & 0x00FF00FFu) | magic;
    }
  }
}

// NVFP4: e2m1 codes of one chunk (4 words, 32 codes) as fp16 pairs worth 2^-14 of their values,
// in the 4-bit pair order: pair 4d + j holds nibbles j and j + 4 of word d. A half's nibble
// s e e m becomes fp16 bits 15 (s) and 11..9 (e e m).
LFM3_DEV void unpack_e2m1(const uint32_t (&w)[4], uint32_t (&p)[16]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = w[d];
    p[4 * d] = ((x & 0x00070007u) << 9) | ((x & 0x00080008u) << 12);
    p[4 * d + 1] = ((x & 0x00700070u) << 5) | ((x & 0x00800080u) << 8);
    p[4 * d + 2] = ((x & 0x07000700u) << 1) | ((x & 0x08000800u) << 4);
    p[4 * d + 3] = ((x & 0x70007000u) >> 3) | (x & 0x80008000u);
  }
}

// Block-FP8: e4m3 codes of one chunk (4 words, 16 codes) as fp16 pairs worth 2^-8 of their
// values, in the 8-bit pair order: pair 2d = bytes 0 and 2 of word d, pair 2d + 1 = bytes 1 and 3.
LFM3_DEV void unpack_e4m3(const uint32_t (&w)[4], uint32_t (&p)[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = w[d], y = w[d] >> 8;
    p[2 * d] = ((x & 0x007F007Fu) << 7) | ((x & 0x00800080u) << 8);
    p[2 * d + 1] = ((y & 0x007F007Fu) << 7) | ((y & 0x00800080u) << 8);
  }
}

LFM3_DEV float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_v, a), __builtin_bit_cast(f16x2_v, b), c, false);
}

// Rows handled together by one wave: 8 for STORE / LOGITS, 4 gate + the 4 matching up rows for
// SWIGLU, B, C and x rows of 2 channels (6, reduced as 8 with two zero rows) for the conv epilogue,
// 2 for STORE2 (outputs too narrow to give every CU a block at 8 rows a wave: out_proj, o_proj and
// qkvg at 2048-3104 rows run 4x the waves, each with a quarter of the dot products).
constexpr int kRG = 8;
template <int EPI> struct RowsPerGroup { static constexpr int v = EPI == GEMV_CONV ? 6 : EPI == GEMV_STORE2 ? 2 : 8; };

template <int EPI> LFM3_HOST_DEV int n_groups_of(int N) {
  if (EPI == GEMV_SWIGLU) return N / 8;
  if (EPI == GEMV_CONV) return N / 6;
  if (EPI == GEMV_STORE2) return (N + 1) / 2;
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
  } else if constexpr (EPI == GEMV_STORE2) {
    rows[0] = 2 * g;
    rows[1] = min(2 * g + 1, N - 1);
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) rows[r] = min(8 * g + r, N - 1);
  }
}

// Sum of 8 per-lane values over the wave, transposed: lanes 8r .. 8r+7 end with the total of
// value r. Cross-half and cross-row exchanges use the gfx950 permlane swaps, the rest DPP; every
// lane evaluates the same addition tree (up to operand order), so the 8 copies are identical and
// the result does not depend on anything but the values.
LFM3_DEV float bfly8(const float (&in)[8]) {
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(in[i]), __float_as_uint(in[i + 4]), false, false);
    v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  float w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 2]), false, false);
    w[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  const bool hi = (threadIdx.x & 8) != 0;
  const float keep = hi ? w[1] : w[0], send = hi ? w[0] : w[1];
  float t = keep + dpp_mov<0x140>(send);  // row_mirror: lane i <-> 15 - i
  t += dpp_mov<0xb1>(t);
  t += dpp_mov<0x4e>(t);
  t += dpp_mov<0x141>(t);                 // row_half_mirror: lane i <-> 7 - i
  return t;
}

// The same for 2 values: lanes 32r .. 32r+31 end with the total of value r (halves swapped by
// permlane32, 16-lane rows by permlane16, then the DPP row sum).
LFM3_DEV float bfly2(float a0, float a1) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
  const float v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return row16_sum(__uint_as_float(q[0]) + __uint_as_float(q[1]));
}

// Stage the fp16 input rows in LDS in chunk pair order with per-chunk sums of the staged values.
// Vector block v (8 consecutive k) lands at fp16 offset 8v, permuted into the order in which the
// unpacked codes pair up.
template <int BITS> LFM3_DEV uint4 pair_order8(const uint32_t (&h)[4]) {
  // h: 8 fp16 in natural order, two per word
  if constexpr (PairOrder<BITS>::v == 4) {
    // (x0, x4), (x1, x5), (x2, x6), (x3, x7)
    return make_uint4(__builtin_amdgcn_perm(h[2], h[0], 0x05040100u), __builtin_amdgcn_perm(h[2], h[0], 0x07060302u),
                      __builtin_amdgcn_perm(h[3], h[1], 0x05040100u), __builtin_amdgcn_perm(h[3], h[1], 0x07060302u));
  } else if constexpr (PairOrder<BITS>::v == 8) {
    // (x0, x2), (x1, x3), (x4, x6), (x5, x7)
    return make_uint4(__builtin_amdgcn_perm(h[1], h[0], 0x05040100u), __builtin_amdgcn_perm(h[1], h[0], 0x07060302u),
                      __builtin_amdgcn_perm(h[3], h[2], 0x05040100u), __builtin_amdgcn_perm(h[3], h[2], 0x07060302u));
  } else {
    return make_uint4(h[0], h[1], h[2], h[3]);
  }
}

// One vector block of one batch row into LDS: the pair-ordered fp16 values and, from the first lane
// of each chunk, the chunk's (X, XO): X = sum of its x, XO = the offset the magic adds to its dot
// products, 1024 * X at 6 and 8 bits and 1024 * X_even + 64 * X_odd at 4 bits (X_even / X_odd:
// the x of the even / odd codes of each 8-code word). Sums: the block's values in order, then the
// lanes of the chunk by a DPP tree.
template <int BITS>
LFM3_DEV void put_x8(uint16_t* xp, float2* xsum, int K, int b, int v, const uint32_t (&h)[4], bool valid) {
  using Q = QT<BITS>;
  float e = 0.f, o = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e += h2f((f16_t)(h[i] & 0xffffu));
    o += h2f((f16_t)(h[i] >> 16));
  }
  e = valid ? e : 0.f;
  o = valid ? o : 0.f;
  e += dpp_mov<0xb1>(e);                    // chunk = 2 vector blocks (16 codes) ...
  o += dpp_mov<0xb1>(o);
  if (Q::CH == 32) { e += dpp_mov<0x4e>(e); o += dpp_mov<0x4e>(o); }   // ... or 4 (32 codes)
  if (!valid) return;
  *(uint4*)(xp + (size_t)b * K + 8 * v) = pair_order8<BITS>(h);
  const float X = e + o;
  const float XO = BITS == 4 ? fmaf(kMagicOff, e, 64.f * o) : kMagicOff * X;
  if ((v & (Q::CH / 8 - 1)) == 0) xsum[b * (K / Q::CH) + v / (Q::CH / 8)] = make_float2(X, XO);
}

// Decode norm prologue registers: the h / m rows of every batch row and the two norm weights.
template <int BT> struct PrologueRegs {
  float hv[BT][kVecBlocks][8], mv[BT][kVecBlocks][8], wpo[kVecBlocks][8], wpr[kVecBlocks][8];
};

// All prologue loads, unconditional (absent inputs read a valid stand-in, masked later), so they
// are issued back to back before the weight prefetch.
template <int BT>
LFM3_DEV void prologue_load(const GemvArgs& a, PrologueRegs<BT>& p) {
  const int K = a.w.k, nv = K / 8;
  const float* mp = a.m ? a.m : a.h_src;
  const bf16_t* wpo = a.w_post ? a.w_post : a.w_pre;
#pragma unroll
  for (int j = 0; j < kVecBlocks; ++j) {
    const int v = min((int)threadIdx.x + 256 * j, nv - 1);
    bf16x8_to_f32(load_u16x8(a.w_pre + 8 * v), p.wpr[j]);
    bf16x8_to_f32(load_u16x8(wpo + 8 * v), p.wpo[j]);
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const size_t o = (size_t)min(b, a.batch - 1) * K + 8 * v;
      load_f32x8(a.h_src + o, p.hv[b][j]);
      load_f32x8(mp + o, p.mv[b][j]);
    }
  }
}

// The norm arithmetic of k_resid_norm (norm_vec.h) per batch row, then the staging. When the input
// is carried as an fp16 pair (split), real row b stages its high parts as virtual row b and its
// remainders as virtual row b + BT/2.
template <int BITS, int BT>
LFM3_DEV void prologue_compute(const GemvArgs& a, PrologueRegs<BT>& p, uint16_t* xp, float2* xsum, float* red,
                               bool split) {
  const int K = a.w.k, nv = K / 8;
  constexpr int HB = BT / 2;
  bool ok[kVecBlocks];
#pragma unroll
  for (int j = 0; j < kVecBlocks; ++j) ok[j] = (int)threadIdx.x + 256 * j < nv;
  const bool first = blockIdx.x == 0;
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    if (split && b >= HB) break;
    if (a.m) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < kVecBlocks; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = ok[j] ? fmaf(p.mv[b][j][e], p.mv[b][j][e], ss) : ss;
      const float rm = rsqrtf(block_sum4(ss, red + 8 * b) / (float)K + a.eps);
#pragma unroll
      for (int j = 0; j < kVecBlocks; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) p.hv[b][j][e] = fmaf(p.mv[b][j][e] * rm, p.wpo[j][e], p.hv[b][j][e]);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kVecBlocks; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = ok[j] ? fmaf(p.hv[b][j][e], p.hv[b][j][e], ss) : ss;
    const float rh = rsqrtf(block_sum4(ss, red + 8 * b + 4) / (float)K + a.eps);
    const bool live = b < a.batch;
#pragma unroll
    for (int j = 0; j < kVecBlocks; ++j) {
      const int v = (int)threadIdx.x + 256 * j;
      float xv[8];
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = (p.hv[b][j][e] * rh) * p.wpr[j][e];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16_t h0 = f2h_sep(xv[2 * e]), h1 = f2h_sep(xv[2 * e + 1]);
        h[e] = live ? ((uint32_t)h0 | ((uint32_t)h1 << 16)) : 0u;
        l[e] = live ? ((uint32_t)f2h_sep(sub_sep(xv[2 * e], h2f(h0))) | ((uint32_t)f2h_sep(sub_sep(xv[2 * e + 1], h2f(h1))) << 16)) : 0u;
      }
      put_x8<BITS>(xp, xsum, K, b, v, h, ok[j]);
      if (split) put_x8<BITS>(xp, xsum, K, b + HB, v, l, ok[j]);
      if (first && live && ok[j]) {
        if (a.m && a.h_dst) store_f32x8(a.h_dst + (size_t)b * K + 8 * v, p.hv[b][j]);
        if (a.capture) store_f32x8(a.capture + (size_t)b * a.capture_ld + 8 * v, p.hv[b][j]);
        if (a.x_copy) store_f32x8(a.x_copy + (size_t)b * K + 8 * v, xv);
      }
    }
  }
}

// Plain fp16 input rows, PVB vector blocks per thread at a time: all loads first, then the
// staging.
template <int BT> struct PlainVB { static constexpr int v = BT <= 2 ? 4 : 2; };
template <int BT> struct PlainRegs { uint4 h[BT][PlainVB<BT>::v]; };

// Virtual row b of a split input reads row b % (BT/2) of x (b < BT/2) or of x_lo.
template <int BT>
LFM3_DEV void plain_load(const GemvArgs& a, PlainRegs<BT>& p, int j0, bool split) {
  const int nv = a.w.k / 8;
  constexpr int HB = BT > 1 ? BT / 2 : 1;
#pragma unroll
  for (int j = 0; j < PlainVB<BT>::v; ++j) {
    const int v = min((int)threadIdx.x + 256 * (j0 + j), nv - 1);
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const int rb = split ? b % HB : b;
      const f16_t* src = (split && b >= HB) ? a.x_lo : a.x;
      p.h[b][j] = load_u16x8(src + (size_t)min(rb, a.batch - 1) * a.ldx + 8 * v);
    }
  }
}

template <int BITS, int BT>
LFM3_DEV void plain_stage(const GemvArgs& a, const PlainRegs<BT>& p, int j0, uint16_t* xp, float2* xsum, bool split) {
  const int K = a.w.k, nv = K / 8;
  constexpr int HB = BT > 1 ? BT / 2 : 1;
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int j = 0; j < PlainVB<BT>::v; ++j) {
      const int v = (int)threadIdx.x + 256 * (j0 + j);
      const bool live = (split ? b % HB : b) < a.batch;
      const uint32_t h[4] = {live ? p.h[b][j].x : 0u, live ? p.h[b][j].y : 0u, live ? p.h[b][j].z : 0u, live ? p.h[b][j].w : 0u};
      put_x8<BITS>(xp, xsum, K, b, v, h, v < nv);
    }
}

// Attention-merge input (PRO = 2, the o_proj of 1-2 rows): thread t stages vector block t (dims
// 8 (t % 16) .. + 7 of head t / 16) of each row from the decode attention's split partials: with
// M the largest split max, x = sigmoid(g) * sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s, the
// online-softmax merge ("LFM3-1.7B port": sigmoid head gate in fp32), rounded to fp16; a row with
// one split takes x as the attention kernel wrote it. Every load (clamped to the row's last split)
// is issued before the weights', the arithmetic after.
template <int BT> struct MergeRegs {
  float4 o[BT][kFusedMergeSplits][2];
  float2 ml[BT][kFusedMergeSplits];
  uint4 xr[BT];
  float g[BT];
};

template <int BT>
LFM3_DEV void merge_load(const GemvArgs& a, MergeRegs<BT>& p) {
  const int nq = a.w.k / kHeadDim;
  const int v = min((int)threadIdx.x, a.w.k / 8 - 1);
  const int h = v >> 4, d0 = 8 * (v & 15);
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const int rb = min(b, a.batch - 1);
    const int ns = a.merge_splits[rb];
    p.g[b] = a.gate_src[(size_t)rb * a.gate_ld + h];
    p.xr[b] = load_u16x8(a.x + (size_t)rb * a.ldx + 8 * v);
    const float* ph = a.part + ((size_t)rb * nq + h) * a.part_splits * kPartStride;
#pragma unroll
    for (int q = 0; q < kFusedMergeSplits; ++q) {
      const float* ps = ph + (size_t)min(q, ns - 1) * kPartStride;
      p.o[b][q][0] = *(const float4*)(ps + d0);
      p.o[b][q][1] = *(const float4*)(ps + d0 + 4);
      p.ml[b][q] = *(const float2*)(ps + kHeadDim);
    }
  }
}

template <int BITS, int BT>
LFM3_DEV void merge_stage(const GemvArgs& a, const MergeRegs<BT>& p, uint16_t* xp, float2* xsum) {
  const int K = a.w.k, v = threadIdx.x;
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const int ns = a.merge_splits[min(b, a.batch - 1)];
    uint32_t hw[4] = {p.xr[b].x, p.xr[b].y, p.xr[b].z, p.xr[b].w};
    if (ns > 1) {
      float mx = p.ml[b][0].x;
#pragma unroll
      for (int q = 1; q < kFusedMergeSplits; ++q) mx = q < ns ? fmaxf(mx, p.ml[b][q].x) : mx;
      float l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < kFusedMergeSplits; ++q) {
        if (q >= ns) continue;
        const float w = __expf(p.ml[b][q].x - mx);
        l = fmaf(w, p.ml[b][q].y, l);
        const float ov[8] = {p.o[b][q][0].x, p.o[b][q][0].y, p.o[b][q][0].z, p.o[b][q][0].w,
                             p.o[b][q][1].x, p.o[b][q][1].y, p.o[b][q][1].z, p.o[b][q][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(w, ov[e], o[e]);
      }
      const float inv = l > 0.f ? (1.f / (1.f + __expf(-p.g[b]))) / l : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) hw[e] = (uint32_t)f2h(o[2 * e] * inv) | ((uint32_t)f2h(o[2 * e + 1] * inv) << 16);
    }
    if (b >= a.batch)
#pragma unroll
      for (int e = 0; e < 4; ++e) hw[e] = 0u;
    put_x8<BITS>(xp, xsum, K, b, v, hw, v < K / 8);
  }
}

// The input: PRO = 0 plain fp16 rows, 1 the decode norm prologue, 2 the attention merge. KW waves
// share one row group (each takes every KW-th k iteration; the partial totals are added in wave
// order through LDS), or KW = 1: each wave owns its groups.
template <int BITS, int BT, int EPI, int PRO, int KW>
__global__ void __launch_bounds__(256) k_gemv(GemvArgs a) {
  using Q = QT<BITS>;
  constexpr int RG = RowsPerGroup<EPI>::v;
  static_assert(EPI != GEMV_STORE2 || KW == 1, "2-row groups are for rows of one wave");
  extern __shared__ uint32_t smem[];
  __shared__ float red[8 * BT];
  __shared__ uint64_t wkeys[EPI == GEMV_LOGITS ? 4 * BT : 1];
  __shared__ float part[KW > 1 ? KW * BT * kRG : 1];
  const int K = a.w.k;
  const int NC = K / Q::CH;
  const int NIT = (NC + 63) / 64;          // k iterations of a group (a multiple of KW)
  const int NITW = NIT / KW;               // of them per wave
  uint16_t* xp = (uint16_t*)smem;                 // [BT][K] fp16 in pair order (virtual rows)
  float2* xsum = (float2*)(smem + (BT * K) / 2);  // [BT][NC] (X, XO)
  // split: the input is carried as an fp16 pair; virtual rows BT/2.. hold the remainders and the
  // two partial totals of a row are added before the epilogue (the host guarantees BT >= 2)
  const bool split = BT > 1 && (a.split_x || a.x_lo);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = a.w.n;
  const int n_groups = n_groups_of<EPI>(N);
  const size_t row_bytes = (size_t)K * Q::CB / 8;
  constexpr bool AFFINE = BITS == 4 || BITS == 6 || BITS == 8;
  const int ngr = AFFINE ? K / a.w.group : 1;
  // group walk: a wave (KW = 1) or a block (KW > 1) takes groups g0, g0 + gstride, ...
  const int g0 = KW == 1 ? blockIdx.x * 4 + wave : blockIdx.x;
  const int gstride = KW == 1 ? gridDim.x * 4 : gridDim.x;
  const int kw = KW == 1 ? 0 : wave;
  const int ngw = g0 < n_groups ? (n_groups - 1 - g0) / gstride + 1 : 0;
  const int nsteps = ngw * NITW;

  // The wave walks a flat sequence of (group, k iteration) steps in two register sets: the first
  // step's weights are requested before the input is staged, the second's before (plain input) or
  // after (norm prologue) the staging, and the load of step s + 2 as soon as step s is computed. Addresses are clamped into range; no step past the
  // wave's last is requested (a spare load of a clamped address still costs its full latency at
  // the end of the wave).
  struct WRegs {
    uint32_t q[RG][Q::NDW];
    bf16_t s[RG], b[RG];   // raw bits: converted when used (NVFP4: s holds the chunk's two e4m3 scales)
    float f[BITS == 48 ? RG : 1];   // block-FP8: the chunk's fp32 block scale
  };
  auto fetch = [&](WRegs& W, int step) {
    const int gi = step / NITW, it = kw + KW * (step - gi * NITW);
    const int c = min(lane + 64 * it, NC - 1);
    int rows[RG];
    rows_of<EPI>(min(g0 + gi * gstride, n_groups - 1), N, rows);
    const int grp = AFFINE ? (c * Q::CH) / a.w.group : 0;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const uint32_t* src = (const uint32_t*)(a.w.q + (size_t)rows[r] * row_bytes + (size_t)c * (Q::CH * Q::CB / 8));
      if constexpr (Q::NDW == 4) {
        const u32x4_v v = __builtin_nontemporal_load((const u32x4_v*)src);
        W.q[r][0] = v[0]; W.q[r][1] = v[1]; W.q[r][2] = v[2]; W.q[r][3] = v[3];
      } else {
#pragma unroll
        for (int d = 0; d < Q::NDW; ++d) W.q[r][d] = __builtin_nontemporal_load(src + d);
      }
      if constexpr (AFFINE) {
        W.s[r] = a.w.scales[(size_t)rows[r] * ngr + grp];
        W.b[r] = a.w.biases[(size_t)rows[r] * ngr + grp];
      } else if constexpr (BITS == 41) {
        W.s[r] = *(const uint16_t*)(a.w.bscale + (size_t)rows[r] * (K / 16) + 2 * c);
      } else if constexpr (BITS == 48) {
        W.f[r] = ((const float*)a.w.bscale)[(size_t)(rows[r] / 128) * ((K + 127) / 128) + (c * Q::CH) / 128];
      }
    }
  };

  // conv epilogue inputs of this wave's first group (taps and kept state of its two channels),
  // loaded with the prologue so that the epilogue has no load of its own for that group
  float cker[EPI == GEMV_CONV ? kMaxTaps : 1], cwin[EPI == GEMV_CONV ? BT : 1][EPI == GEMV_CONV ? kMaxTaps : 1];
  auto conv_prefetch = [&]() {
    if constexpr (EPI == GEMV_CONV) {
      const int H = N / 3, T = a.conv_taps, S = T - 1;
      const int ch = min(2 * min(g0, n_groups - 1) + ((lane >> 3) & 1), H - 1);
#pragma unroll
      for (int q = 0; q < kMaxTaps; ++q) cker[q] = bf2f(a.conv_kernel[(size_t)ch * T + min(q, T - 1)]);
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const f16_t* st = a.conv_state + (size_t)a.conv_slot[min(b, a.batch - 1)] * a.conv_slot_stride;
#pragma unroll
        for (int q = 0; q < kMaxTaps - 1; ++q) cwin[b][q] = h2f(st[(size_t)min(q, S - 1) * H + ch]);
      }
    }
  };

  WRegs wa, wb;
  if constexpr (PRO == 1) {
    // prologue loads first, then the first step's weights, then the prologue arithmetic (the
    // in-order load counter lets the weights stay in flight through it), then the second step's
    // weights (requested before the arithmetic, they measured slower: the prologue is the longer
    // path)
    PrologueRegs<BT> p;
    prologue_load<BT>(a, p);
    conv_prefetch();
    __builtin_amdgcn_sched_barrier(0);
    fetch(wa, 0);
    __builtin_amdgcn_sched_barrier(0);
    prologue_compute<BITS, BT>(a, p, xp, xsum, red, split);
    if (nsteps > 1) fetch(wb, 1);
  } else if constexpr (PRO == 2) {
    MergeRegs<BT> mr;
    merge_load<BT>(a, mr);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    fetch(wa, 0);
    if (nsteps > 1) fetch(wb, 1);
    __builtin_amdgcn_sched_barrier(0);
    merge_stage<BITS, BT>(a, mr, xp, xsum);
  } else {
    // (a barrier without a wait: every wave of the block has its input loads queued before any
    // wave queues weight loads behind them)
    PlainRegs<BT> p;
    plain_load<BT>(a, p, 0, split);
    conv_prefetch();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    fetch(wa, 0);
    if (nsteps > 1) fetch(wb, 1);
    __builtin_amdgcn_sched_barrier(0);
    plain_stage<BITS, BT>(a, p, 0, xp, xsum, split);
    for (int j0 = PlainVB<BT>::v; 256 * j0 < K / 8; j0 += PlainVB<BT>::v) {
      plain_load<BT>(a, p, j0, split);
      plain_stage<BITS, BT>(a, p, j0, xp, xsum, split);
    }
  }
  __syncthreads();

  // the magic exponent in a VGPR (opaque to constant folding), so that the unpack's and-or can take
  // its mask from an SGPR
  uint32_t vmagic = kMagic2;
  asm volatile("" : "+v"(vmagic));

  uint64_t best[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) best[b] = 0;
  float acc[kRG][BT];
#pragma unroll
  for (int r = 0; r < kRG; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;

  auto consume = [&](const WRegs& W, int step) {
    const int gi = step / NITW, sw = step - gi * NITW;
    const int c = lane + 64 * (kw + KW * sw);
    if (c < NC) {
      uint32_t xv[BT][Q::NP];
      float X[BT], XO[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const uint4* xs4 = (const uint4*)(xp + b * K + c * Q::CH);
#pragma unroll
        for (int q = 0; q < Q::NP / 4; ++q) {
          const uint4 v = xs4[q];
          xv[b][4 * q] = v.x; xv[b][4 * q + 1] = v.y; xv[b][4 * q + 2] = v.z; xv[b][4 * q + 3] = v.w;
        }
        const float2 xs = xsum[b * NC + c];
        X[b] = xs.x;
        XO[b] = xs.y;
      }
      if constexpr (BITS == 16) {
        // stored bf16 weights: products of exact fp32 values (8 + 11 significant bits), fp32 sums
        float xf[BT][8];
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            xf[b][2 * q] = h2f((f16_t)(xv[b][q] & 0xffffu));
            xf[b][2 * q + 1] = h2f((f16_t)(xv[b][q] >> 16));
          }
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            float d = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              d = fmaf(__uint_as_float(W.q[r][q] << 16), xf[b][2 * q], d);
              d = fmaf(__uint_as_float(W.q[r][q] & 0xffff0000u), xf[b][2 * q + 1], d);
            }
            acc[r][b] += d;
          }
      } else if constexpr (BITS == 41) {
        // NVFP4: two groups of 16 codes a chunk (pairs 0-7, 8-15), each times its e4m3 scale; the
        // values carry 2^-14 (codes) and 2^-8 (scales), removed with the tensor scale at the end
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          uint32_t wp[16];
          unpack_e2m1(W.q[r], wp);
          const float s0 = h2f((f16_t)e4m3_f16_scaled(W.s[r] & 0xffu)), s1 = h2f((f16_t)e4m3_f16_scaled(W.s[r] >> 8));
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              d0 = dot2(wp[p], xv[b][p], d0);
              d1 = dot2(wp[p + 8], xv[b][p + 8], d1);
            }
            acc[r][b] += fmaf(d0, s0, d1 * s1);
          }
        }
      } else if constexpr (BITS == 48) {
        // block-FP8: one fp32 scale for the chunk; the values carry 2^-8, removed at the end
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          uint32_t wp[8];
          unpack_e4m3(W.q[r], wp);
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            float d = 0.f;
#pragma unroll
            for (int p = 0; p < 8; ++p) d = dot2(wp[p], xv[b][p], d);
            acc[r][b] = fmaf(d, W.f[r], acc[r][b]);
          }
        }
      } else {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        uint32_t wp[Q::NP];
        unpack<BITS>(W.q[r], wp, vmagic);
        const float sc = bf2f(W.s[r]), bi = bf2f(W.b[r]);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          float inner;
          if constexpr (BITS == 4) {
            // even pairs carry 1024 + q, odd pairs 1024 + 16 q
            float da = 0.f, db = 0.f;
#pragma unroll
            for (int p = 0; p < Q::NP; p += 2) {
              da = dot2(wp[p], xv[b][p], da);
              db = dot2(wp[p + 1], xv[b][p + 1], db);
            }
            inner = fmaf(db, 0.0625f, da) - XO[b];
          } else {
            float d = 0.f;
#pragma unroll
            for (int p = 0; p < Q::NP; ++p) d = dot2(wp[p], xv[b][p], d);
            inner = d - XO[b];
          }
          acc[r][b] += fmaf(sc, inner, bi * X[b]);
        }
      }
      }
    }
    if (sw != NITW - 1) return;
    const int g = g0 + gi * gstride;
    // t[b]: lanes 8r .. 8r+7 (2-row groups: 32r .. 32r+31) hold the total of row r of the group
    float t[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      if constexpr (RG == 2) {
        t[b] = bfly2(acc[0][b], acc[1][b]);
      } else {
        float v8[8];
#pragma unroll
        for (int r = 0; r < kRG; ++r) v8[r] = acc[r][b];
        t[b] = bfly8(v8);
      }
    }
#pragma unroll
    for (int r = 0; r < kRG; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;
    if constexpr (KW > 1) {
      if ((lane & 7) == 0)
#pragma unroll
        for (int b = 0; b < BT; ++b) part[(wave * BT + b) * kRG + (lane >> 3)] = t[b];
      __syncthreads();
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        float s = part[b * kRG + (lane >> 3)];
#pragma unroll
        for (int w = 1; w < KW; ++w) s += part[(w * BT + b) * kRG + (lane >> 3)];
        t[b] = s;
      }
      __syncthreads();
      if (wave != 0) return;
    }
    if constexpr (BT > 1) {
      if (split)
#pragma unroll
        for (int b = 0; b < BT / 2; ++b) t[b] = t[b] + t[b + BT / 2];
    }
    if constexpr (BITS == 41 || BITS == 48) {
      // the codes' and scales' powers of two (2^-14 and 2^-8, or 2^-8), and NVFP4's tensor scale
      const float mult = BITS == 41 ? a.w.tscale * 4194304.f : 256.f;
#pragma unroll
      for (int b = 0; b < BT; ++b) t[b] *= mult;
    }
    const int r = lane >> 3;
    if constexpr (EPI == GEMV_STORE) {
      if ((lane & 7) == 0 && 8 * g + r < N)
#pragma unroll
        for (int b = 0; b < BT; ++b)
          if (b < a.batch) a.yf[(size_t)b * a.ldy + 8 * g + r] = t[b];
    } else if constexpr (EPI == GEMV_STORE2) {
      const int n = 2 * g + (lane >> 5);
      if ((lane & 31) == 0 && n < N)
#pragma unroll
        for (int b = 0; b < BT; ++b)
          if (b < a.batch) a.yf[(size_t)b * a.ldy + n] = t[b];
    } else if constexpr (EPI == GEMV_SWIGLU) {
      // silu(a) * b is rounded to fp32, then to fp16, in every batch-size instance, so a row's
      // result does not depend on the batch it is decoded in
      float up[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) up[b] = __shfl_xor(t[b], 32, 64);
      if ((lane & 7) == 0 && r < 4)
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b >= a.batch) continue;
          const float gt = t[b];
          const float sv = gt / (1.f + __expf(-gt)) * up[b];
          a.y[(size_t)b * a.ldy + 4 * g + r] = f2h_sep(sv);
        }
    } else if constexpr (EPI == GEMV_CONV) {
      // gated short conv of channels 2g, 2g+1 ("LFM3-1.7B port" table row 1): z = f16(B * x),
      // y = sum_j ker[c, j] * [state | z]_j, out = f16(C * y), state <- last taps-1 z.
      // Rows: B of the two channels in lanes 0 / 8, C in 16 / 24, x in 32 / 40.
      float cg[BT], xg[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) { cg[b] = __shfl(t[b], (lane + 16) & 63, 64); xg[b] = __shfl(t[b], (lane + 32) & 63, 64); }
      if ((lane & 7) == 0 && r < 2) {
        const int H = N / 3, T = a.conv_taps, S = T - 1;
        const int ch = 2 * g + r;
        const bool pre = gi == 0;   // the first group's taps and state were loaded up front
        float ker[kMaxTaps];
#pragma unroll
        for (int q = 0; q < kMaxTaps; ++q) ker[q] = pre ? cker[q] : (q < T ? bf2f(a.conv_kernel[(size_t)ch * T + q]) : 0.f);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b >= a.batch) continue;
          f16_t* st = a.conv_state + (size_t)a.conv_slot[b] * a.conv_slot_stride;
          const float z = h2f(f2h_sep(t[b] * xg[b]));
          float win[kMaxTaps];
#pragma unroll
          for (int q = 0; q < kMaxTaps - 1; ++q) win[q] = pre ? cwin[b][q] : (q < S ? h2f(st[(size_t)q * H + ch]) : 0.f);
          float kS = ker[kMaxTaps - 1];
#pragma unroll
          for (int q = kMaxTaps - 2; q >= 0; --q) kS = (q == S) ? ker[q] : kS;   // ker[S]
          float y = kS * z;
#pragma unroll
          for (int q = 0; q < kMaxTaps - 1; ++q)
            if (q < S) y = fmaf(ker[q], win[q], y);
#pragma unroll
          for (int q = 0; q < kMaxTaps - 2; ++q)
            if (q + 1 < S) st[(size_t)q * H + ch] = f2h(win[q + 1]);
          st[(size_t)(S - 1) * H + ch] = f2h(z);
          a.y[(size_t)b * a.ldy + ch] = f2h_sep(cg[b] * y);
        }
      }
    } else {
      const int n = 8 * g + r;
      if ((lane & 7) == 0 && n < N)
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b >= a.batch) continue;
          if (a.logits) a.logits[(size_t)b * a.ld_logits + n] = t[b];
          const uint64_t key = ((uint64_t)order_key(t[b]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)n);
          best[b] = key > best[b] ? key : best[b];
        }
    }
  };

  for (int step = 0; step < nsteps; step += 2) {
    consume(wa, step);
    if (step + 2 < nsteps) fetch(wa, step + 2);
    if (step + 1 < nsteps) {
      consume(wb, step + 1);
      if (step + 3 < nsteps) fetch(wb, step + 3);
    }
  }
  if constexpr (EPI == GEMV_LOGITS) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      uint64_t k = best[b];
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, o, 64), hi = __shfl_xor((uint32_t)(k >> 32), o, 64);
        const uint64_t other = ((uint64_t)hi << 32) | lo;
        k = other > k ? other : k;
      }
      if (lane == 0) wkeys[wave * BT + b] = k;
    }
    // the block's best key per row, in one plain store to the row's partial slot
    __syncthreads();
    if ((int)threadIdx.x < BT && (int)threadIdx.x < a.batch) {
      const int b = threadIdx.x;
      uint64_t k = wkeys[b];
#pragma unroll
      for (int w = 1; w < 4; ++w) k = wkeys[w * BT + b] > k ? wkeys[w * BT + b] : k;
      a.keys[(size_t)b * kArgmaxParts + blockIdx.x] = k;
    }
  }
}

#ifndef LFM3_GEMV_MAX_BLOCKS
#define LFM3_GEMV_MAX_BLOCKS 256
#endif

template <int BITS, int BT, int PRO, int KW>
static void launch_epi(hipStream_t s, const GemvArgs& a, int epi, int grid, size_t lds) {
  if constexpr (KW == 1) {
    if (epi == GEMV_STORE2) {
      hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE2, PRO, KW>), dim3(grid), dim3(256), lds, s, a);
      return;
    }
  }
  if constexpr (BITS == 41 || BITS == 48) {
    // the FFN formats: w13 with the SwiGLU epilogue, w2 plain (the caller refuses other epilogues)
    if (epi == GEMV_SWIGLU) hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_SWIGLU, PRO, KW>), dim3(grid), dim3(256), lds, s, a);
    else hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE, PRO, KW>), dim3(grid), dim3(256), lds, s, a);
    return;
  }
  switch (epi) {
    case GEMV_STORE: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE, PRO, KW>), dim3(grid), dim3(256), lds, s, a); break;
    case GEMV_SWIGLU: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_SWIGLU, PRO, KW>), dim3(grid), dim3(256), lds, s, a); break;
    case GEMV_CONV: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_CONV, PRO, KW>), dim3(grid), dim3(256), lds, s, a); break;
    default: hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_LOGITS, PRO, KW>), dim3(grid), dim3(256), lds, s, a); break;
  }
}

template <int BITS, int BT>
static hipError_t launch_bt(hipStream_t s, const GemvArgs& a) {
  using Q = QT<BITS>;
  const int K = a.w.k;
  const size_t lds = (size_t)BT * K * 2 + (size_t)BT * (K / Q::CH) * sizeof(float2);
  const int N = a.w.n;
  int epi = a.epi;
  int n_groups = epi == GEMV_SWIGLU ? n_groups_of<GEMV_SWIGLU>(N)
                 : epi == GEMV_CONV ? n_groups_of<GEMV_CONV>(N) : n_groups_of<GEMV_STORE>(N);
  // Long rows (4 or more k iterations of 64 chunks) are shared by the 4 waves of a block, so that
  // narrow matrices still spread over the whole chip.
  const int nit = (K / Q::CH + 63) / 64;
  const bool split = nit % 4 == 0;
  // a block per 4 row groups (one per wave), or per group when its 4 waves share the group's K
  // range, at most one block per CU; the head (147 MB at 4 bits, bandwidth-bound) takes two blocks
  // per CU for more loads in flight. Waves with more groups than one walk them in steps.
  const int cap = a.max_blocks > 0 ? a.max_blocks : (epi == GEMV_LOGITS ? 2 * LFM3_GEMV_MAX_BLOCKS : LFM3_GEMV_MAX_BLOCKS);
  // plain outputs whose 8-row groups would leave CUs without a block take 2-row groups
  if (epi == GEMV_STORE && !split && (n_groups + 3) / 4 < cap) {
    epi = GEMV_STORE2;
    n_groups = n_groups_of<GEMV_STORE2>(N);
  }
  int grid = split ? n_groups : (n_groups + 3) / 4;
  if (grid > cap) grid = cap;
  if (a.epi == GEMV_LOGITS && grid > kArgmaxParts) return hipErrorInvalidValue;
  if (a.h_src) {
    if constexpr (BT <= 2) {
      if (split) launch_epi<BITS, BT, 1, 4>(s, a, epi, grid, lds);
      else launch_epi<BITS, BT, 1, 1>(s, a, epi, grid, lds);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (a.part) {
    if constexpr (BT <= 2) {
      if (a.epi != GEMV_STORE) return hipErrorInvalidValue;
      if (split) hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE, 2, 4>), dim3(grid), dim3(256), lds, s, a);
      else if (epi == GEMV_STORE2) hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE2, 2, 1>), dim3(grid), dim3(256), lds, s, a);
      else hipLaunchKernelGGL((k_gemv<BITS, BT, GEMV_STORE, 2, 1>), dim3(grid), dim3(256), lds, s, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    if (split) launch_epi<BITS, BT, 0, 4>(s, a, epi, grid, lds);
    else launch_epi<BITS, BT, 0, 1>(s, a, epi, grid, lds);
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_bits(hipStream_t s, const GemvArgs& a) {
  using Q = QT<BITS>;
  const int K = a.w.k;
  auto lds_for = [&](int bt) { return (size_t)bt * K * 2 + (size_t)bt * (K / Q::CH) * sizeof(float2); };
  // a split input takes two virtual rows per row
  const bool split = a.split_x || a.x_lo;
  const int rows = split ? 2 * a.batch : a.batch;
  int bt = rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : 8;
  while (bt > (split ? 2 : 1) && lds_for(bt) > 65536) bt >>= 1;
  if (split && a.split_x && 2 * a.batch > bt) return hipErrorInvalidValue;   // prologue: one launch
  if ((split ? 2 * a.batch : a.batch) > bt) {
    const int per = split ? bt / 2 : bt;
    // split the batch into launches of at most bt rows (plain x input only)
    if (a.h_src) return hipErrorInvalidValue;
    for (int b0 = 0; b0 < a.batch; b0 += per) {
      GemvArgs p = a;
      p.batch = a.batch - b0 < per ? a.batch - b0 : per;
      p.x = a.x + (size_t)b0 * a.ldx;
      if (p.x_lo) p.x_lo = a.x_lo + (size_t)b0 * a.ldx;
      for (int i = 0; i < p.batch; ++i) p.conv_slot[i] = a.conv_slot[b0 + i];
      if (p.y) p.y = a.y + (size_t)b0 * a.ldy;
      if (p.yf) p.yf = a.yf + (size_t)b0 * a.ldy;
      if (p.logits) p.logits = a.logits + (size_t)b0 * a.ld_logits;
      if (p.keys) p.keys = a.keys + (size_t)b0 * kArgmaxParts;
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
  if (a.epi < GEMV_STORE || a.epi > GEMV_CONV) return hipErrorInvalidValue;   // STORE2 is picked here, not asked for
  // attention-merge input: one vector block per thread, whole heads, 1-2 rows of at most
  // kFusedMergeSplits splits, plain STORE
  if (a.part) {
    if (a.h_src || a.x_lo || a.split_x || a.epi != GEMV_STORE || a.batch > 2 || a.w.k > 256 * 8 ||
        a.w.k % kHeadDim || !a.gate_src || !a.x || a.part_splits < 1)
      return hipErrorInvalidValue;
    for (int b = 0; b < a.batch; ++b)
      if (a.merge_splits[b] < 1 || a.merge_splits[b] > kFusedMergeSplits || a.merge_splits[b] > a.part_splits)
        return hipErrorInvalidValue;
  }
  // vector staging: rows of 8-element blocks, 16-byte aligned; the norm prologue takes K <= 4096
  if (a.w.k % 8 || (a.h_src && a.w.k > 256 * 8 * kVecBlocks)) return hipErrorInvalidValue;
  if (a.h_src ? ((uintptr_t)a.h_src % 16 || (a.m && (uintptr_t)a.m % 16) || (uintptr_t)a.w_pre % 16 ||
                 (a.w_post && (uintptr_t)a.w_post % 16))
              : ((uintptr_t)a.x % 16 || a.ldx % 8 || (uintptr_t)a.x_lo % 16))
    return hipErrorInvalidValue;
  switch (a.w.fmt) {
    case FMT_AFFINE:
      switch (a.w.bits) {
        case 4: return launch_bits<4>(s, a);
        case 6: return launch_bits<6>(s, a);
        case 8: return launch_bits<8>(s, a);
        default: return hipErrorInvalidValue;
      }
    case FMT_BF16: return launch_bits<16>(s, a);
    case FMT_NVFP4:
      if (a.w.k % 32 || (a.epi != GEMV_STORE && a.epi != GEMV_SWIGLU) || a.part) return hipErrorInvalidValue;
      return launch_bits<41>(s, a);
    case FMT_FP8B:
      if (a.w.k % 16 || (a.epi != GEMV_STORE && a.epi != GEMV_SWIGLU) || a.part) return hipErrorInvalidValue;
      return launch_bits<48>(s, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lfm3
