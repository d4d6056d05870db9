// Small per-row kernels of the LFM3 forward pass on gfx950: embedding gather, residual + sandwich
// RMSNorm, per-head q/k norm + RoPE + KV store, the gated short conv with its kept state, and
// bookkeeping (page table, argmax finalisation, fills, the dequant check).
#include "kernels.h"
#include "norm_vec.h"

namespace lfm3 {

// Code k of a row stored as a little-endian low-bit-first bitstream of `bits`-bit codes.
LFM3_DEV uint32_t code_at(const uint8_t* row, int k, int bits) {
  const int bit = k * bits;
  const int byte = bit >> 3, sh = bit & 7;
  uint32_t v = row[byte];
  if (sh + bits > 8) v |= (uint32_t)row[byte + 1] << 8;
  return (v >> sh) & ((1u << bits) - 1u);
}

// The affine dequantisation w = q * scale + bias (MLX affine format); exact in fp32 for bf16
// scale/bias and codes below 2^8.
LFM3_DEV float deq_value(uint32_t q, float s, float b) { return fmaf((float)q, s, b); }

// ---------------------------------------------------------------------------------------------
// embedding ("LFM3-1.7B port" table: vocab 128000, tied; TensorFold #1491: quantized like the
// linears, 8-bit in the VL 4-bit export)
// ---------------------------------------------------------------------------------------------

// Block (row, 256-column slice), one column per thread: the whole row's loads go out at once (one
// block looping over the row waited for each slice's loads in turn: 6 us a decode step at batch 1).
__global__ void __launch_bounds__(256) k_embed(QLinear e, const int32_t* __restrict__ tokens, float* __restrict__ h,
                                                uint32_t* flags) {
  const int r = blockIdx.x;
  const int k = blockIdx.y * blockDim.x + threadIdx.x;
  const int tok = tokens[r];
  if (k >= e.k) return;
  float* out = h + (size_t)r * e.k;
  if (tok < 0 || tok >= e.n) {
    out[k] = 0.f;
    if (k == 0) atomicOr(flags, 1u);
    return;
  }
  if (e.fmt != FMT_AFFINE) {
    out[k] = weight_value(e, tok, k);
    return;
  }
  const size_t row_bytes = (size_t)e.k * e.bits / 8;
  const uint8_t* row = e.q + (size_t)tok * row_bytes;
  const int ng = e.k / e.group;
  const int g = k / e.group;
  const float s = bf2f(e.scales[(size_t)tok * ng + g]);
  const float b = bf2f(e.biases[(size_t)tok * ng + g]);
  out[k] = deq_value(code_at(row, k, e.bits), s, b);
}

hipError_t launch_embed(hipStream_t s, const QLinear& emb, const int32_t* tokens, int rows, float* h, uint32_t* flags) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_embed, dim3(rows, (emb.k + 255) / 256), dim3(256), 0, s, emb, tokens, h, flags);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) k_bf16_to_f32(const bf16_t* __restrict__ in, size_t n, float* __restrict__ out) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) out[i] = bf2f(in[i]);
}

hipError_t launch_bf16_to_f32(hipStream_t s, const bf16_t* in, int rows, int cols, float* out) {
  const size_t n = (size_t)rows * cols;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_bf16_to_f32, dim3((unsigned)blocks), dim3(256), 0, s, in, n, out);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) k_dequant_rows(QLinear w, int row0, float* f32, f16_t* hv) {
  const int r = blockIdx.x;
  const int n = row0 + r;
  if (w.fmt != FMT_AFFINE) {
    for (int k = threadIdx.x; k < w.k; k += blockDim.x) {
      const float v = weight_value(w, n, k);
      if (f32) f32[(size_t)r * w.k + k] = v;
      if (hv) hv[(size_t)r * w.k + k] = f2h(v);
    }
    return;
  }
  const size_t row_bytes = (size_t)w.k * w.bits / 8;
  const uint8_t* row = w.q + (size_t)n * row_bytes;
  const int ng = w.k / w.group;
  for (int k = threadIdx.x; k < w.k; k += blockDim.x) {
    const int g = k / w.group;
    const float v = deq_value(code_at(row, k, w.bits), bf2f(w.scales[(size_t)n * ng + g]),
                              bf2f(w.biases[(size_t)n * ng + g]));
    if (f32) f32[(size_t)r * w.k + k] = v;
    if (hv) hv[(size_t)r * w.k + k] = f2h(v);
  }
}

hipError_t launch_dequant_rows(hipStream_t s, const QLinear& w, int row0, int rows, float* f32, f16_t* h) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequant_rows, dim3(rows), dim3(256), 0, s, w, row0, f32, h);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// residual + sandwich RMSNorm ("LFM3-1.7B port" table row 5: operator_norm -> mixer ->
// post_operator_norm -> + residual -> ffn_norm -> SwiGLU -> post_ffn_norm -> + residual;
// RMSNorm eps 1e-5). One block per row, 256 threads, hidden <= 4096.
// ---------------------------------------------------------------------------------------------

// NP: partial sums of m the row carries (1: m; 2: m + m2, the prefill K halves; 4: m + m2 + m3 + m4,
// the decode K quarters). Every partial is loaded with the first loads: loaded behind a runtime
// test, each one waited for the one before it.
template <int NP>
__global__ void __launch_bounds__(256) k_resid_norm(NormArgs a) {
  // the arithmetic is the decode GEMV's norm prologue (norm_vec.h), so fused and unfused steps
  // agree bitwise
  __shared__ float red[8];
  const int r = blockIdx.x;
  const int H = a.hidden;
  const size_t base = (size_t)r * H;
  const int nv = H / 8;
  float hv[kVecBlocks][8], mv[kVecBlocks][8], wpo[kVecBlocks][8], wpr[kVecBlocks][8];
  float pv[NP > 1 ? NP - 1 : 1][kVecBlocks][8];
  const float* mp = a.m ? a.m : a.h_in;
  const float* pp[3] = {a.m2, a.m3, a.m4};
  const bf16_t* wpo_p = a.w_post ? a.w_post : a.w_pre;
#pragma unroll
  for (int j = 0; j < kVecBlocks; ++j) {
    const int v = min((int)threadIdx.x + 256 * j, nv - 1);
    load_f32x8(a.h_in + base + 8 * v, hv[j]);
    load_f32x8(mp + base + 8 * v, mv[j]);
#pragma unroll
    for (int q = 0; q + 1 < NP; ++q) load_f32x8(pp[q] + base + 8 * v, pv[q][j]);
    bf16x8_to_f32(load_u16x8(wpo_p + 8 * v), wpo[j]);
    bf16x8_to_f32(load_u16x8(a.w_pre + 8 * v), wpr[j]);
  }
  if constexpr (NP > 1) {
#pragma unroll
    for (int j = 0; j < kVecBlocks; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mv[j][e] = mv[j][e] + pv[0][j][e];
        if constexpr (NP == 4) mv[j][e] = (mv[j][e] + pv[1][j][e]) + pv[2][j][e];
      }
  }
  bool ok[kVecBlocks];
#pragma unroll
  for (int j = 0; j < kVecBlocks; ++j) ok[j] = (int)threadIdx.x + 256 * j < nv;
  if (a.m) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kVecBlocks; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = ok[j] ? fmaf(mv[j][e], mv[j][e], ss) : ss;
    const float rm = rsqrtf(block_sum4(ss, red) / (float)H + a.eps);
#pragma unroll
    for (int j = 0; j < kVecBlocks; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[j][e] = fmaf(mv[j][e] * rm, wpo[j][e], hv[j][e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kVecBlocks; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = ok[j] ? fmaf(hv[j][e], hv[j][e], ss) : ss;
  const float rh = rsqrtf(block_sum4(ss, red + 4) / (float)H + a.eps);
#pragma unroll
  for (int j = 0; j < kVecBlocks; ++j) {
    if (!ok[j]) continue;
    const int k = 8 * ((int)threadIdx.x + 256 * j);
    float xv[8];
    uint32_t xh[4], xl[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = (hv[j][e] * rh) * wpr[j][e];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f16_t h0 = f2h_sep(xv[2 * e]), h1 = f2h_sep(xv[2 * e + 1]);
      xh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      xl[e] = (uint32_t)f2h_sep(sub_sep(xv[2 * e], h2f(h0))) | ((uint32_t)f2h_sep(sub_sep(xv[2 * e + 1], h2f(h1))) << 16);
    }
    if (a.x_lo) *(uint4*)(a.x_lo + base + k) = make_uint4(xl[0], xl[1], xl[2], xl[3]);
    if (a.m) store_f32x8(a.h_out + base + k, hv[j]);
    if (a.capture) store_f32x8(a.capture + base + k, hv[j]);
    if (a.x_copy) store_f32x8(a.x_copy + base + k, xv);
    *(uint4*)(a.x_out + base + k) = make_uint4(xh[0], xh[1], xh[2], xh[3]);
  }
}

hipError_t launch_resid_norm(hipStream_t s, const NormArgs& a) {
  if (a.rows <= 0) return hipSuccess;
  // the partials present (a partial without m is never passed; m3 and m4 come together)
  if (!a.m || !a.m2) hipLaunchKernelGGL(k_resid_norm<1>, dim3(a.rows), dim3(256), 0, s, a);
  else if (!a.m3) hipLaunchKernelGGL(k_resid_norm<2>, dim3(a.rows), dim3(256), 0, s, a);
  else if (a.m4) hipLaunchKernelGGL(k_resid_norm<4>, dim3(a.rows), dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// q/k per-head RMSNorm, RoPE and the KV store.
// "LFM3-1.7B port": per-head q/k RMSNorm unchanged from LFM2.5; "partial_rotary_factor" section:
// rotate_half pairs (i, i+64), angle p * inv_freq_i, inv_freq 0 on the tail of the full layers.
// One block per row, 4 waves; lane l holds dims l and l + 64 of a head.
// ---------------------------------------------------------------------------------------------

LFM3_DEV f16_t* kv_row(const KvRef& kv, f16_t* base, int slot, int pos, int kvh, int n_kv) {
  if (kv.ring == 0) {
    const int page = kv.page_table[(size_t)slot * kv.max_pages + pos / kPageTokens];
    return base + (((size_t)page * n_kv + kvh) * kPageTokens + (pos % kPageTokens)) * kHeadDim;
  }
  return base + (((size_t)slot * n_kv + kvh) * kv.ring + (pos % kv.ring)) * kHeadDim;
}

__global__ void __launch_bounds__(256) k_qk_rope(QkRopeArgs a) {
  const int r = blockIdx.x;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int pos = row_pos(a.rows, r), slot = row_slot(a.rows, r);
  const float* src = a.qkvg + (size_t)r * a.ld;
  const float c = a.cos_t[(size_t)pos * kHalfDim + l];
  const float sn = a.sin_t[(size_t)pos * kHalfDim + l];
  const int nq = a.n_q_heads, nkv = a.n_kv_heads;
  // q heads and k heads: norm + rope
  for (int h = w; h < nq + nkv; h += 4) {
    const bool is_q = h < nq;
    const float* hp = src + (size_t)h * kHeadDim;  // k heads follow q heads contiguously
    const float x0 = hp[l], x1 = hp[l + kHalfDim];
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float rr = rsqrtf(ss / (float)kHeadDim + a.eps);
    const bf16_t* nw = is_q ? a.q_norm : a.k_norm;
    const float n0 = x0 * rr * bf2f(nw[l]);
    const float n1 = x1 * rr * bf2f(nw[l + kHalfDim]);
    const float o0 = n0 * c - n1 * sn;
    const float o1 = n1 * c + n0 * sn;
    f16_t* dst;
    if (is_q) {
      dst = a.q_out + ((size_t)r * nq + h) * kHeadDim;
    } else {
      dst = kv_row(a.kv, a.kv.k, slot, pos, h - nq, nkv);
    }
    dst[l] = f2h(o0);
    dst[l + kHalfDim] = f2h(o1);
  }
  // v heads: stored fp16 as produced
  for (int h = w; h < nkv; h += 4) {
    const float* vp = src + (size_t)(nq + nkv + h) * kHeadDim;
    f16_t* dst = kv_row(a.kv, a.kv.v, slot, pos, h, nkv);
    dst[l] = f2h(vp[l]);
    dst[l + kHalfDim] = f2h(vp[l + kHalfDim]);
  }
}

hipError_t launch_qk_rope(hipStream_t s, const QkRopeArgs& a) {
  if (a.rows.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_qk_rope, dim3(a.rows.n), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Keys and values of positions [p0, p0 + n) of one slot between the cache (pool pages or the
// slot's ring) and contiguous buffers kbuf / vbuf [n, n_kv, 128]: a kept state's save (dir 0,
// cache -> buffer) and load (dir 1). Block per position; thread t < 64 moves 16-byte chunk t of
// the key row, t >= 64 chunk t - 64 of the value row.
__global__ void __launch_bounds__(128) k_kv_move(KvRef kv, int slot, int p0, f16_t* kbuf, f16_t* vbuf, int n_kv,
                                                 int dir) {
  const int i = blockIdx.x, t = threadIdx.x;
  const int pos = p0 + i;
  const bool is_k = t < 64;
  const int c = (t & 63) * 8;   // element offset within the n_kv * 128 row
  const int h = c / kHeadDim, e = c % kHeadDim;
  f16_t* cache = kv_row(kv, is_k ? kv.k : kv.v, slot, pos, h, n_kv) + e;
  f16_t* buf = (is_k ? kbuf : vbuf) + ((size_t)i * n_kv + h) * kHeadDim + e;
  if (dir == 0) *(uint4*)buf = *(const uint4*)cache;
  else *(uint4*)cache = *(const uint4*)buf;
}

hipError_t launch_kv_move(hipStream_t s, const KvRef& kv, int slot, int p0, int n, f16_t* kbuf, f16_t* vbuf, int n_kv,
                          int dir) {
  if (n <= 0) return hipSuccess;
  if (n_kv * kHeadDim != 512) return hipErrorInvalidValue;   // 64 chunks of 8 per key row
  hipLaunchKernelGGL(k_kv_move, dim3(n), dim3(128), 0, s, kv, slot, p0, kbuf, vbuf, n_kv, dir);
  return hipGetLastError();
}

__global__ void k_copy16(uint4* dst, const uint4* src, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) dst[i] = src[i];
}

hipError_t launch_copy(hipStream_t s, void* dst, const void* src, size_t bytes) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 || (uintptr_t)dst % 16 || (uintptr_t)src % 16) return hipErrorInvalidValue;
  const size_t n = bytes / 16;
  size_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_copy16, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)dst, (const uint4*)src, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// gated short conv ("LFM3-1.7B port" table row 1: kernel 7, state = last 6 columns of B*x;
// "--pad-tail": the new state is columns [n, n + 6) of [state | Bx] after n real rows).
// Prefill (rows.mode 0): block (channel block, row block); the row-block-0 block alone reads and
// then rewrites the slot's state, so no other block races with it. Decode (mode 1): one block per
// row, each row a distinct slot.
// ---------------------------------------------------------------------------------------------

constexpr int kConvRun = 8;   // prefill rows per thread

__global__ void __launch_bounds__(256) k_conv(ConvArgs a) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= a.hidden) return;
  const int H = a.hidden, T = a.taps, S = T - 1;
  // taps past T read tap T - 1 and are zeroed after the load: clamped addresses keep every load
  // unconditional, so they all go out at once (a guarded load per tap waited for each in turn)
  auto load_taps = [&](bf16_t (&kraw)[kMaxTaps]) {
#pragma unroll
    for (int j = 0; j < kMaxTaps; ++j) kraw[j] = a.kernel[(size_t)c * T + min(j, T - 1)];
  };
  auto zrow = [&](int r) -> float {
    const float* p = a.bcx + (size_t)r * a.ld;
    return h2f(f2h_sep(p[c] * p[2 * H + c]));
  };
  float ker[kMaxTaps];
  bf16_t kraw[kMaxTaps];
  if (a.rows.mode == 1) {
    // the row's own loads (state columns, B, C, x) go out first, then the taps; the tap loops run
    // to the compile-time bound so the window stays in registers. The sums are those of in_proj's
    // fused conv epilogue: z first, then the state columns oldest first.
    const int r = blockIdx.y;
    f16_t* st = a.state + (size_t)a.rows.slot[r] * a.slot_stride;
    f16_t sraw[kMaxTaps - 1];
#pragma unroll
    for (int j = 0; j < kMaxTaps - 1; ++j) sraw[j] = st[(size_t)min(j, S - 1) * H + c];
    const float* p = a.bcx + (size_t)r * a.ld;
    const float bv = p[c], cv = p[H + c], xv = p[2 * H + c];
    load_taps(kraw);
    float win[kMaxTaps - 1];
#pragma unroll
    for (int j = 0; j < kMaxTaps - 1; ++j) win[j] = j < S ? h2f(sraw[j]) : 0.f;
    const float z = h2f(f2h_sep(bv * xv));
#pragma unroll
    for (int j = 0; j < kMaxTaps; ++j) ker[j] = j < T ? bf2f(kraw[j]) : 0.f;
    float kS = ker[kMaxTaps - 1];
#pragma unroll
    for (int q = kMaxTaps - 2; q >= 0; --q) kS = q == S ? ker[q] : kS;   // ker[S]
    float y = kS * z;
#pragma unroll
    for (int j = 0; j < kMaxTaps - 1; ++j)
      if (j < S) y = fmaf(ker[j], win[j], y);
    a.out[(size_t)r * H + c] = f2h_sep(cv * y);
#pragma unroll
    for (int j = 0; j < kMaxTaps - 2; ++j)
      if (j + 1 < S) st[(size_t)j * H + c] = f2h(win[j + 1]);
    st[(size_t)(S - 1) * H + c] = f2h(z);
    return;
  }
  load_taps(kraw);
#pragma unroll
  for (int j = 0; j < kMaxTaps; ++j) ker[j] = j < T ? bf2f(kraw[j]) : 0.f;
  // prefill: a run of kConvRun rows of one channel per thread; every input of the run (z of the
  // run and of the taps-1 rows before it, from bcx or, before row 0, the kept state; C of the run)
  // is loaded up front (clamped addresses, branch-free), then the run is computed
  const int M = a.rows.n;
  const int r0 = blockIdx.y * kConvRun;
  f16_t* st = a.state + (size_t)a.rows.slot0 * a.slot_stride;
  constexpr int NZ = kConvRun + kMaxTaps - 1;
  float bz[NZ], xz[NZ], sz[NZ], cz[kConvRun];
#pragma unroll
  for (int i = 0; i < NZ; ++i) {
    const int t = r0 - S + i;
    const int tt = min(max(t, 0), M - 1);
    const float* p = a.bcx + (size_t)tt * a.ld;
    bz[i] = p[c];
    xz[i] = p[2 * H + c];
    sz[i] = h2f(st[(size_t)min(max(S + t, 0), S - 1) * H + c]);
  }
#pragma unroll
  for (int i = 0; i < kConvRun; ++i) cz[i] = a.bcx[(size_t)min(r0 + i, M - 1) * a.ld + H + c];
  float z[NZ];
#pragma unroll
  for (int i = 0; i < NZ; ++i) z[i] = (r0 - S + i) < 0 ? sz[i] : h2f(f2h_sep(bz[i] * xz[i]));
  // z[i + S] is row r0 + i; the taps before it are z[i] .. z[i + S - 1] (all indices constant
  // after unrolling, selected by S)
  const float kS = bf2f(a.kernel[(size_t)c * T + S]);
#pragma unroll
  for (int i = 0; i < kConvRun; ++i) {
    const int r = r0 + i;
    float zc = z[i + kMaxTaps - 1];
#pragma unroll
    for (int q = kMaxTaps - 2; q >= 0; --q) zc = (q + 1 == S) ? z[i + q + 1] : zc;   // z[i + S]
    float y = kS * zc;
#pragma unroll
    for (int j = 0; j < kMaxTaps - 1; ++j)
      if (j < S) y = fmaf(ker[j], z[i + j], y);
    if (r < M) {
      a.out[(size_t)r * H + c] = f2h_sep(cz[i] * y);
      if (a.z_out) a.z_out[(size_t)r * H + c] = f2h(zc);
    }
  }
  if (blockIdx.y == 0) {
    // new state: the last S entries of [state | z_0 .. z_{M-1}]; ascending j reads state[M + j]
    // (M >= 1) before it is overwritten, and no other block reads the state.
    for (int j = 0; j < S; ++j) {
      const int t = M - S + j;
      const float v = t >= 0 ? zrow(t) : h2f(st[(size_t)(S + t) * H + c]);
      st[(size_t)j * H + c] = f2h(v);
    }
  }
}

hipError_t launch_conv(hipStream_t s, const ConvArgs& a) {
  if (a.rows.n <= 0) return hipSuccess;
  const int cb = (a.hidden + 255) / 256;
  if (a.taps > kMaxTaps || a.taps < 2 || a.hidden % 256) return hipErrorInvalidValue;
  const int rb = a.rows.mode == 1 ? a.rows.n : (a.rows.n + kConvRun - 1) / kConvRun;
  hipLaunchKernelGGL(k_conv, dim3(cb, rb), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Verify-window commit ("TensorFold PR #1508": the commit of an accepted row's conv state): block
// (channel block, conv layer).
__global__ void __launch_bounds__(256) k_conv_commit(f16_t* state, const f16_t* pre, const f16_t* z, int zrows,
                                                     int accept, int hidden, int S) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int l = blockIdx.y;
  if (c >= hidden) return;
  const f16_t* pl = pre + (size_t)l * S * hidden;
  const f16_t* zl = z + (size_t)l * zrows * hidden;
  f16_t* st = state + (size_t)l * S * hidden;
  for (int j = 0; j < S; ++j) {
    const int w = accept + j;   // index into [pre (S columns) | z_0 .. z_{accept-1}]
    st[(size_t)j * hidden + c] = w < S ? pl[(size_t)w * hidden + c] : zl[(size_t)(w - S) * hidden + c];
  }
}

hipError_t launch_conv_commit(hipStream_t s, f16_t* state, const f16_t* pre, const f16_t* z, int zrows, int accept,
                              int n_conv, int hidden, int taps) {
  if (n_conv <= 0) return hipSuccess;
  if (accept < 0 || accept > zrows || taps < 2 || taps > kMaxTaps) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_conv_commit, dim3((hidden + 255) / 256, n_conv), dim3(256), 0, s, state, pre, z, zrows, accept,
                     hidden, taps - 1);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// bookkeeping
// ---------------------------------------------------------------------------------------------

struct PageList { int32_t v[32]; };

__global__ void k_set_pages(int32_t* pt, int index0, int count, PageList pl) {
  const int i = threadIdx.x;
  if (i < count) pt[index0 + i] = pl.v[i];
}

hipError_t launch_set_pages(hipStream_t s, int32_t* page_table, int index0, int count, const int32_t* pages) {
  for (int off = 0; off < count; off += 32) {
    PageList pl;
    const int n = count - off < 32 ? count - off : 32;
    for (int i = 0; i < n; ++i) pl.v[i] = pages[off + i];
    hipLaunchKernelGGL(k_set_pages, dim3(1), dim3(32), 0, s, page_table, index0 + off, n, pl);
  }
  return hipGetLastError();
}

__global__ void k_zero(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_zero(hipStream_t s, void* p, size_t bytes) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, n);
  return hipGetLastError();
}

// keys: (order_key(value) << 32) | (0xffffffff - index); the max key is the largest value with
// the lowest index. Block r takes the kArgmaxParts partials of row r (max is order-free, so the
// result does not depend on which block wrote which part) and clears them for the next step.
__global__ void __launch_bounds__(256) k_argmax_finalize(uint64_t* keys, int32_t* ids) {
  __shared__ uint64_t wk[4];
  const int r = blockIdx.x;
  uint64_t* part = keys + (size_t)r * kArgmaxParts;
  // every partial of the thread is loaded before any is cleared (a load after a store to the same
  // array would wait for it)
  static_assert(kArgmaxParts % 256 == 0, "whole partials per thread");
  constexpr int kPer = kArgmaxParts / 256;
  uint64_t v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) v[i] = part[threadIdx.x + 256 * i];
  uint64_t k = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    k = v[i] > k ? v[i] : k;
    part[threadIdx.x + 256 * i] = 0;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)k, o, 64), hi = __shfl_xor((uint32_t)(k >> 32), o, 64);
    const uint64_t other = ((uint64_t)hi << 32) | lo;
    k = other > k ? other : k;
  }
  if ((threadIdx.x & 63) == 0) wk[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0 && ids) {
    k = wk[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) k = wk[w] > k ? wk[w] : k;
    ids[r] = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffu));
  }
}

hipError_t launch_argmax_finalize(hipStream_t s, uint64_t* keys, int32_t* ids, int rows) {
  if (rows <= 0) return hipSuccess;
  if (rows > kMaxBatch) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_argmax_finalize, dim3(rows), dim3(256), 0, s, keys, ids);
  return hipGetLastError();
}

}  // namespace lfm3
