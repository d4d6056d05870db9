// Host-side launchers of the gfx950 LFM3 kernels. All launch on the given stream and return the
// launch status; shapes are validated by the caller (runtime.hip) before any launch.
#pragma once
#include "common.h"

namespace lfm3 {

// ---- k_misc.hip ------------------------------------------------------------------------------

// h[r, :] = q * scale + bias (fp32, exact) of embedding row tokens[r]; an id outside [0, vocab)
// gives a zero row and sets bit 0 of *flags (a device word the host reads at its next sync).
hipError_t launch_embed(hipStream_t s, const QLinear& emb, const int32_t* tokens, int rows, float* h, uint32_t* flags);
// h[r, :] = float(bf16 input row)
hipError_t launch_bf16_to_f32(hipStream_t s, const bf16_t* in, int rows, int cols, float* out);

// Residual + sandwich norm, one row per block; the residual stream h and the mixer/FFN output m
// are fp32, the normed matmul input x is fp16:
//   if m:  h_out = h_in + rmsnorm(m) * w_post   else h_out = h_in (may alias)
//   x_out = f16(rmsnorm(h_out) * w_pre)
// capture (nullable) receives h_out; x_copy (nullable) receives rmsnorm(h_out) * w_pre in fp32.
struct NormArgs {
  const float* h_in;
  const float* m;
  const float* m2;  // nullable: the mixer/FFN output is m + m2 (two K-half partials, added in that order)
  const float* m3;  // nullable (with m2): four K-quarter partials, added as ((m + m2) + m3) + m4
  const float* m4;
  const bf16_t* w_post;
  const bf16_t* w_pre;
  float* h_out;
  f16_t* x_out;
  f16_t* x_lo;      // nullable: the fp16 remainder x - f16(x), so x_out + x_lo carries x to ~22 bits
  float* capture;
  float* x_copy;
  int rows, hidden;
  float eps;
};
hipError_t launch_resid_norm(hipStream_t s, const NormArgs& a);

// Where attention K/V live: full layers in pool pages through the slot page table, sliding layers
// in a per-slot ring of `ring` rows indexed by position mod ring.
struct KvRef {
  f16_t* k;            // fp16 keys after norm + RoPE
  f16_t* v;            // fp16 values
  const int32_t* page_table;  // full: [max_slots, max_pages]
  int32_t max_pages;
  int32_t ring;               // sliding: rows per slot ring (0 for paged)
};

// Per-head q/k RMSNorm + RoPE (pairs (i, i+64) with cos/sin tables [max_ctx, 64]); q to q_out
// [rows, 16, 128]; k, v into the cache at each row's (slot, position).
struct QkRopeArgs {
  const float* qkvg;   // [rows, ld]: q | k | v | g (fp32 linear output)
  int ld;
  const bf16_t* q_norm;
  const bf16_t* k_norm;
  const float* cos_t;
  const float* sin_t;
  f16_t* q_out;
  KvRef kv;
  Rows rows;
  int n_q_heads, n_kv_heads;
  float eps;
};
hipError_t launch_qk_rope(hipStream_t s, const QkRopeArgs& a);

// Gated short conv with kept state: z = f16(B*x); y = sum_j ker[c, j] * [state | z]_j;
// out = f16(C * y); state <- last (taps-1) z. bcx [rows, ld] holds B | C | x (fp32).
struct ConvArgs {
  const float* bcx;
  int ld;
  const bf16_t* kernel;  // [hidden, taps]
  f16_t* state;          // this layer's state of slot 0: [taps-1, hidden]; slot stride below
  int64_t slot_stride;
  f16_t* out;            // [rows, hidden]
  f16_t* z_out;          // nullable (prefill): every row's z = f16(B * x), [rows, hidden], for a
                         // verify window's commit
  Rows rows;
  int hidden, taps;
};
hipError_t launch_conv(hipStream_t s, const ConvArgs& a);
// Commit of a verify window's accepted rows: each conv layer's state of one slot becomes the last
// taps - 1 columns of [pre | z_0 .. z_{accept-1}], where pre is the state before the window
// ([n_conv, taps-1, hidden]) and z the window rows' z ([n_conv, zrows, hidden]).
hipError_t launch_conv_commit(hipStream_t s, f16_t* state, const f16_t* pre, const f16_t* z, int zrows, int accept,
                              int n_conv, int hidden, int taps);

// Keys and values of positions [p0, p0 + n) of `slot` between the cache and contiguous fp16
// buffers [n, n_kv, 128] (dir 0: save, cache -> buffers; 1: load, buffers -> cache). n_kv = 4.
hipError_t launch_kv_move(hipStream_t s, const KvRef& kv, int slot, int p0, int n, f16_t* kbuf, f16_t* vbuf, int n_kv,
                          int dir);
// Device-to-device copy of `bytes` (16-byte multiple, 16-byte aligned) by a kernel.
hipError_t launch_copy(hipStream_t s, void* dst, const void* src, size_t bytes);
hipError_t launch_set_pages(hipStream_t s, int32_t* page_table, int index0, int count, const int32_t* pages);
hipError_t launch_zero(hipStream_t s, void* p, size_t bytes);
hipError_t launch_argmax_finalize(hipStream_t s, uint64_t* keys, int32_t* ids, int rows);
hipError_t launch_dequant_rows(hipStream_t s, const QLinear& w, int row0, int rows, float* f32, f16_t* h);

// ---- k_gemv.hip --------------------------------------------------------------------------------

enum GemvEpi { GEMV_STORE = 0, GEMV_SWIGLU = 1, GEMV_LOGITS = 2, GEMV_CONV = 3,
               GEMV_STORE2 = 4 };   // STORE in 2-row groups: chosen by launch_gemv itself for narrow outputs
// y[b, n] = sum_k x[b, k] * (q[n, k] * s + bias) for b < batch (<= 8), exact weights (the per-group
// factored form). STORE: fp32 yf [batch, ldy]. SWIGLU: rows n and n + N/2 -> fp16 silu(a) * b in
// y. LOGITS: fp32 logits (nullable) + per-block argmax partials (keys, kArgmaxParts per row). CONV (in_proj, N = 3H): the
// gated short conv of each channel with its kept state, fp16 out in y [batch, ldy].
// Input: x fp16 [batch, ldx], or (h_src set) the decode norm prologue:
//   h_new = h_src + (m ? rmsnorm(m) * w_post : 0), x = f16(rmsnorm(h_new) * w_pre),
// with block 0 writing h_new to h_dst (when m is set), capture rows and the fp32 x copy.
struct GemvArgs {
  QLinear w;
  const f16_t* x;   // [batch, ldx]
  const f16_t* x_lo;  // nullable, [batch, ldx]: fp16 remainder of x (input carried as x + x_lo)
  int ldx;
  int split_x;      // norm prologue: carry x as the fp16 pair x_hi + x_lo
  int batch;
  int epi;
  f16_t* y;
  float* yf;
  int ldy;
  float* logits;
  int ld_logits;
  uint64_t* keys;
  // norm prologue (rows of length K, contiguous)
  const float* h_src;
  const float* m;
  const bf16_t* w_post;
  const bf16_t* w_pre;
  float eps;
  float* h_dst;
  float* capture;
  int capture_ld;
  float* x_copy;
  // conv epilogue
  const bf16_t* conv_kernel;  // [H, taps]
  f16_t* conv_state;          // this layer's state of slot 0; slot stride below
  int64_t conv_slot_stride;
  int conv_taps;
  int32_t conv_slot[kMaxBatch];
  int max_blocks;             // grid cap (0: default)
  // decode MFMA GEMM, STORE epilogue (nullable): K split in four quarters run by separate blocks;
  // quarter 0's sums go to yf, quarters 1..3's to yf_part[0..2] (the consumer adds them in order)
  float* yf_part[3];
  // attention-merge input (o_proj at 1-2 rows; part nullable): x row b is the gated merge of row
  // b's decode-attention split partials ([batch, K / 128 heads, part_splits, kPartStride]) when
  // merge_splits[b] > 1, else x itself (the attention kernel's gated output of a one-split row);
  // the gate logit of head h of row b is gate_src[b * gate_ld + h]. At most kFusedMergeSplits
  // splits a row, K <= 2048, no norm prologue.
  const float* part;
  int part_splits;
  const float* gate_src;
  int gate_ld;
  int32_t merge_splits[kMaxBatch];
};
hipError_t launch_gemv(hipStream_t s, const GemvArgs& a);

// ---- k_gemm.hip --------------------------------------------------------------------------------

enum GemmEpi { GEMM_STORE = 0, GEMM_SWIGLU = 1 };

// A quantized linear re-tiled for the prefill GEMM (built once from the blob's linear by
// launch_repack_gemm). Tile (t, kt) covers weight rows [32t, 32t + 32) (rows past N repeat row
// N - 1) and k [64kt, 64kt + 64); lane l of a wave holds row 32t + l % 32, k 64kt + 32(l / 32) ..
// + 31: its codes (16 B at 4-bit, 32 B at 8-bit as two 16-byte planes, 24 B at 6-bit as three
// 8-byte planes; each plane is 64 lanes contiguous) and one dword of fp16 (scale, bias) for its
// group. 4-bit codes are reordered inside each 32-bit word (code j of the word at nibble
// 0, 2, 4, 6, 1, 3, 5, 7 for j = 0 .. 7) so that the byte-permute unpack yields k in order.
//
// w16 (nullable) holds the same weights already dequantised, f16(q * s + bias) computed exactly as
// the GEMM's register dequantisation does, in its operand order: per tile, plane t (t = 0 .. 3) is
// 64 lanes x 16 B, lane l's 8 fp16 weights of row 32t' + l % 32 at k 64kt + 32(l / 32) + 8t .. +7.
// The prefill GEMM reads it when present (no dequantisation work in the K loop; 4x the bytes of
// 4-bit codes), else it dequantises the codes.
struct GemmW {
  const uint8_t* codes;
  const uint32_t* sb;
  const uint32_t* w16;
  int32_t n, k, bits, group, ntile;
  int32_t fmt;   // the stored format (WeightFmt); bf16, NVFP4 and block-FP8 have only w16
};
size_t gemm_codes_bytes(int n, int k, int bits);
size_t gemm_sb_bytes(int n, int k);
size_t gemm_w16_bytes(int n, int k);
hipError_t launch_repack_gemm(hipStream_t s, const QLinear& w, uint8_t* codes, uint32_t* sb);
// w16 from the re-tiled codes and (scale, bias) of w (which must already hold them).
hipError_t launch_repack_gemm16(hipStream_t s, const GemmW& w, uint32_t* w16);
// w16 straight from a linear stored as bf16, NVFP4 or block-FP8: f16 of each weight's fp32 value
// (weight_value), in the same operand order. These linears have no re-tiled codes.
hipError_t launch_make_w16(hipStream_t s, const QLinear& w, uint32_t* w16);

// Decode linears of 3 .. 32 rows on MFMA from the re-tiled weights: the GEMV's STORE, SWIGLU,
// CONV and LOGITS epilogues with its argument block (x, x_lo, batch, outputs, conv state, argmax
// keys); the input rows (x, and x_lo as extra rows when set) number at most 64.
hipError_t launch_sgemm(hipStream_t s, const GemmW& w, const GemvArgs& g);
// Whether launch_sgemm splits a STORE linear's K in four (when the caller passes yf_part).
inline bool sgemm_store_ksplit(const GemmW& w) { return w.ntile < 128 && (w.k / 64) % 4 == 0 && w.k / 64 >= 32; }

// Y[m, n] = sum_k X[m, k] * f16(q[n, k] * s + bias), MFMA fp16 with fp32 accumulation.
// STORE writes fp32 yf; SWIGLU writes fp16 y.
struct GemmArgs {
  GemmW w;
  const f16_t* x;   // [M, ldx]
  const f16_t* x_lo;  // nullable, [M, ldx]: fp16 remainder of x; Y = (x + x_lo) W as two K passes
  int ldx;
  int m;
  int epi;
  f16_t* y;         // [M, ldy]
  float* yf;
  float* yf2;       // nullable (STORE, no x_lo): K is split in two halves run by separate blocks; the
                    // first half's sums go to yf, the second half's to yf2 (the consumer adds them)
  int ldy;
};
hipError_t launch_gemm(hipStream_t s, const GemmArgs& a);

// ---- k_attn.hip --------------------------------------------------------------------------------

// Causal (full) or sliding-window attention over the cache for a pass's rows; output gated by
// sigmoid(g) per head and stored fp16 [rows, n_q_heads * 128].
struct AttnArgs {
  const f16_t* q;      // [rows, n_q_heads, 128] (after norm + RoPE)
  const float* gate;   // [rows, ldg] (g columns, fp32 linear output)
  int ldg;
  KvRef kv;
  Rows rows;
  int window;          // 0 = full causal
  int n_q_heads, n_kv_heads;
  f16_t* out;          // [rows, n_q_heads * 128]
  float* part;         // split-K partials (decode)
  int max_splits;
};
hipError_t launch_attn_prefill(hipStream_t s, const AttnArgs& a);

// Decode attention for one row per slot, fused with the q/k norm + RoPE of the step's own query
// and key and the store of its key and value; split-K (attn_decode_split_keys keys per split) with
// the partials merged by a second launch.
struct AttnDecodeArgs {
  const float* qkvg;   // raw fp32 linear output [rows, ld]: q | k | v | g
  int ld;
  int gate_col;        // column of g_0
  const bf16_t* q_norm;
  const bf16_t* k_norm;
  const float* cos_t;
  const float* sin_t;
  KvRef kv;
  Rows rows;
  int window;          // 0 = full causal
  int n_q_heads, n_kv_heads;
  float eps;
  f16_t* out;          // [rows, n_q_heads * 128]
  float* part;         // [rows, n_q_heads, max_splits, kPartStride]
  int max_splits;      // grid extent: the most splits any row needs
  int merge_in_consumer;   // the next linear merges the partials itself (no merge launch)
};
constexpr int kPartStride = kHeadDim + 4;   // split partial: o [128], max, sum, 2 pad (16-byte rows)
constexpr int kFusedMergeSplits = 4;        // most splits per row the o_proj GEMV merges itself
hipError_t launch_attn_decode(hipStream_t s, const AttnDecodeArgs& a);

// Keys per split of a decode row with `keys` visible keys: one 64-key tile per split (a block per
// tile runs in parallel) while that gives at most 64 splits, beyond that the keys in 64 equal
// splits of whole tiles, so a long row is at most 64 blocks per kv head and its merge reads at most
// 64 partials; sliding layers always take single tiles. It depends on the row alone, which keeps a
// row's result independent of the batch it is decoded in.
LFM3_HOST_DEV int attn_decode_split_keys(bool sliding, int keys) {
  if (sliding) return 64;
  const int s = ((keys + 63) / 64 + 63) / 64 * 64;
  return s > 64 ? s : 64;
}

}  // namespace lfm3
