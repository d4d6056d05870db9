// Host runtime and C ABI of the LFM3 forward pass: config and blob admission, workspace layout,
// slot bookkeeping (lengths, KV pages), and the layer walk for prefill passes and decode steps.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/lfm3.h"
#include "kernels.h"

using namespace lfm3;

namespace {

thread_local std::string g_err;

constexpr int kMaxVerify = 16;   // rows of a verify window

// ------------------------------------------------------------------------------------------------
// blob format (the writer is the seeded input generator; this reader is independent)
//   64-byte header: "LFM3BLB1", u32 version 1, u32 n_tensors, u64 table_offset, u64 data_offset,
//   u64 total_bytes; then n_tensors 128-byte entries: name[80], u32 dtype, u32 ndim, u32 shape[4],
//   u64 offset, u64 nbytes. dtype 0 = packed codes (bytes), 1 = bf16.
// ------------------------------------------------------------------------------------------------
struct Entry {
  uint32_t dtype, ndim, shape[4];
  uint64_t offset, nbytes;
};

constexpr uint32_t DT_CODES = 0, DT_BF16 = 1, DT_F32 = 2;

// Storage of one linear: format, code bits, group (affine) -- from the config by role.
struct LinFmt {
  int fmt, bits, group;
};
enum LinRole { ROLE_MIXER = 0, ROLE_FFN = 1, ROLE_EMBED = 2 };
LinFmt fmt_of(const lfm3_config& c, int role) {
  if (role == ROLE_EMBED) return c.embed_bits == 16 ? LinFmt{FMT_BF16, 16, 0} : LinFmt{FMT_AFFINE, c.embed_bits, c.embed_group};
  if (role == ROLE_FFN && c.ffn_format == LFM3_FFN_NVFP4) return {FMT_NVFP4, 4, 16};
  if (role == ROLE_FFN && c.ffn_format == LFM3_FFN_FP8_BLOCK) return {FMT_FP8B, 8, 128};
  return c.bits == 16 ? LinFmt{FMT_BF16, 16, 0} : LinFmt{FMT_AFFINE, c.bits, c.group};
}

struct Expect {
  std::string name;
  uint32_t dtype;
  std::vector<uint32_t> shape;
};

int n_of_type(const lfm3_config& c, int t) {
  int n = 0;
  for (int i = 0; i < c.n_layers; ++i) n += c.layer_type[i] == t;
  return n;
}

int qkvg_rows(const lfm3_config& c) { return c.n_q_heads * c.head_dim + 2 * c.n_kv_heads * c.head_dim + c.n_q_heads; }

void add_linear(std::vector<Expect>& v, const std::string& name, uint32_t n, uint32_t k, LinFmt f) {
  if (f.fmt == FMT_BF16) {
    v.push_back({name + ".weight", DT_BF16, {n, k}});
  } else if (f.fmt == FMT_NVFP4) {
    v.push_back({name + ".fp4", DT_CODES, {n, k / 2}});
    v.push_back({name + ".block_scales", DT_CODES, {n, k / 16}});
    v.push_back({name + ".tensor_scale", DT_F32, {1}});
    v.push_back({name + ".input_scale", DT_F32, {1}});
  } else if (f.fmt == FMT_FP8B) {
    v.push_back({name + ".fp8", DT_CODES, {n, k}});
    v.push_back({name + ".block_scales", DT_F32, {(n + 127) / 128, (k + 127) / 128}});
  } else {
    v.push_back({name + ".q", DT_CODES, {n, (uint32_t)((uint64_t)k * f.bits / 8)}});
    v.push_back({name + ".scales", DT_BF16, {n, k / (uint32_t)f.group}});
    v.push_back({name + ".biases", DT_BF16, {n, k / (uint32_t)f.group}});
  }
}

std::vector<Expect> expected_tensors(const lfm3_config& c) {
  std::vector<Expect> v;
  const uint32_t H = c.hidden, F = c.ffn, D = c.head_dim;
  const LinFmt fm = fmt_of(c, ROLE_MIXER), ff = fmt_of(c, ROLE_FFN);
  if (c.has_embedding) add_linear(v, "embedding", c.vocab, H, fmt_of(c, ROLE_EMBED));
  for (int i = 0; i < c.n_layers; ++i) {
    const std::string p = "layers." + std::to_string(i) + ".";
    for (const char* nm : {"operator_norm", "post_operator_norm", "ffn_norm", "post_ffn_norm"})
      v.push_back({p + nm, DT_BF16, {H}});
    if (c.layer_type[i] == LFM3_LAYER_CONV) {
      v.push_back({p + "conv.kernel", DT_BF16, {H, (uint32_t)c.conv_taps}});
      add_linear(v, p + "conv.in_proj", 3 * H, H, fm);
      add_linear(v, p + "conv.out_proj", H, H, fm);
    } else {
      v.push_back({p + "attn.q_norm", DT_BF16, {D}});
      v.push_back({p + "attn.k_norm", DT_BF16, {D}});
      add_linear(v, p + "attn.qkvg_proj", qkvg_rows(c), H, fm);
      add_linear(v, p + "attn.o_proj", H, c.n_q_heads * D, fm);
    }
    add_linear(v, p + "ffn.w13", 2 * F, H, ff);
    add_linear(v, p + "ffn.w2", H, F, ff);
  }
  v.push_back({"embedding_norm", DT_BF16, {H}});
  return v;
}

uint64_t elem_bytes(const Expect& e) {
  uint64_t n = e.dtype == DT_BF16 ? 2 : e.dtype == DT_F32 ? 4 : 1;
  for (uint32_t s : e.shape) n *= s;
  return n;
}

bool parse_header(const uint8_t* p, size_t bytes, std::unordered_map<std::string, Entry>& out, uint64_t& total, std::string& err) {
  if (bytes < 64) { err = "blob smaller than its 64-byte header"; return false; }
  if (memcmp(p, "LFM3BLB1", 8) != 0) { err = "blob magic is not LFM3BLB1"; return false; }
  uint32_t ver, n;
  uint64_t tab, dat;
  memcpy(&ver, p + 8, 4); memcpy(&n, p + 12, 4); memcpy(&tab, p + 16, 8); memcpy(&dat, p + 24, 8); memcpy(&total, p + 32, 8);
  if (ver != 1) { err = "blob version " + std::to_string(ver) + " is not 1"; return false; }
  if (tab + (uint64_t)n * 128 > bytes || tab + (uint64_t)n * 128 > dat) { err = "blob tensor table runs past the data offset"; return false; }
  for (uint32_t i = 0; i < n; ++i) {
    const uint8_t* e = p + tab + (uint64_t)i * 128;
    char name[81];
    memcpy(name, e, 80);
    name[80] = 0;
    Entry en;
    memcpy(&en.dtype, e + 80, 4); memcpy(&en.ndim, e + 84, 4); memcpy(en.shape, e + 88, 16);
    memcpy(&en.offset, e + 104, 8); memcpy(&en.nbytes, e + 112, 8);
    if (out.count(name)) { err = std::string("blob names tensor ") + name + " twice"; return false; }
    out[name] = en;
  }
  return true;
}

bool check_config(const lfm3_config& c, std::string& err) {
  auto bad = [&](const char* f, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, f);
    vsnprintf(buf, sizeof buf, f, ap);
    va_end(ap);
    err = buf;
    return false;
  };
  if (c.n_layers < 1 || c.n_layers > LFM3_MAX_LAYERS) return bad("n_layers %d outside [1, %d]", c.n_layers, LFM3_MAX_LAYERS);
  if (c.hidden < 512 || c.hidden > 4096 || c.hidden % 512) return bad("hidden %d: this build runs multiples of 512 up to 4096", c.hidden);
  if (c.ffn < 512 || c.ffn % 512) return bad("ffn %d: this build runs multiples of 512", c.ffn);
  if (c.head_dim != kHeadDim) return bad("head_dim %d: this build runs 128", c.head_dim);
  if (c.n_kv_heads < 1 || c.n_q_heads != kQPerKv * c.n_kv_heads) return bad("heads %d/%d: this build runs 4 query heads per KV head", c.n_q_heads, c.n_kv_heads);
  if (c.n_q_heads * c.head_dim != c.hidden) return bad("n_q_heads * head_dim %d != hidden %d", c.n_q_heads * c.head_dim, c.hidden);
  if (c.vocab < 1) return bad("vocab %d", c.vocab);
  if (c.conv_taps < 2 || c.conv_taps > kMaxTaps) return bad("conv_taps %d outside [2, %d]", c.conv_taps, kMaxTaps);
  if (c.window < 1) return bad("window %d", c.window);
  if (c.rope_pairs_full < 0 || c.rope_pairs_full > kHalfDim || c.rope_pairs_sliding < 0 || c.rope_pairs_sliding > kHalfDim)
    return bad("rope pairs %d/%d outside [0, 64]", c.rope_pairs_full, c.rope_pairs_sliding);
  if (!(c.rope_theta_full > 1.0) || !(c.rope_theta_sliding > 1.0)) return bad("rope theta must be > 1 (full %g, sliding %g)", c.rope_theta_full, c.rope_theta_sliding);
  if (!(c.norm_eps > 0.f)) return bad("norm_eps must be > 0");
  auto bits_ok = [](int b) { return b == 4 || b == 6 || b == 8 || b == 16; };
  if (!bits_ok(c.bits)) return bad("unsupported affine bits %d (4, 6 or 8; 16 for stored bf16)", c.bits);
  if (c.bits != 16 && c.group != 32 && c.group != 64) return bad("unsupported affine group %d (32 or 64)", c.group);
  if (c.has_embedding != 0 && c.has_embedding != 1) return bad("has_embedding must be 0 or 1");
  if (c.has_embedding) {
    if (!bits_ok(c.embed_bits)) return bad("unsupported embedding bits %d", c.embed_bits);
    if (c.embed_bits != 16 && c.embed_group != 32 && c.embed_group != 64) return bad("unsupported embedding group %d", c.embed_group);
  }
  if (c.ffn_format < LFM3_FFN_AS_LINEARS || c.ffn_format > LFM3_FFN_FP8_BLOCK)
    return bad("unsupported ffn_format %d (0 as the other linears, 1 NVFP4, 2 block-FP8)", c.ffn_format);
  for (int i = 0; i < c.n_layers; ++i)
    if (c.layer_type[i] > LFM3_LAYER_SLIDING) return bad("layer %d has unknown type %d", i, c.layer_type[i]);
  if (c.max_slots < 1) return bad("max_slots %d", c.max_slots);
  // max_ctx sizes the RoPE tables and the page-table rows; 65536 is the largest context validated here
  if (c.max_ctx < 1 || c.max_ctx > 65536) return bad("max_ctx %d outside [1, 65536]", c.max_ctx);
  if (c.page_tokens != kPageTokens) return bad("page_tokens %d: this build runs 16", c.page_tokens);
  if (c.max_chunk < 1) return bad("max_chunk %d", c.max_chunk);
  if (c.n_pages < 0) return bad("n_pages %d", c.n_pages);
  if (n_of_type(c, LFM3_LAYER_FULL) > 0 && c.n_pages < 1) return bad("full-attention layers need n_pages >= 1");
  return true;
}

// ------------------------------------------------------------------------------------------------
// workspace layout
// ------------------------------------------------------------------------------------------------
struct Layout {
  size_t cos_f, sin_f, cos_s, sin_s;
  size_t conv_state, ring_k, ring_v, pool_k, pool_v, page_table;
  size_t h, h2, x, xlo, big, sbuf, mix, qrot, m, m2, m3, m4, xf, part, keys, flags;
  size_t vpre, vz;   // verify windows: each slot's conv state before its window, and the window rows' z
  size_t gemm_w, gemm_w_bytes;   // re-tiled copies of every prefill GEMM weight
  size_t total;
  int max_rows, max_pages, ring_rows, max_splits, big_ld;
  size_t ring_layer, pool_layer, conv_slot;
};

// (N, K) of every prefill GEMM weight, in layer order: the mixer's input and output linears, then
// w13 and w2.
// (N, K, role) of every prefill GEMM weight, in layer order: the mixer's input and output linears,
// then w13 and w2.
struct GemmShape {
  int n, k, role;
};
std::vector<GemmShape> gemm_shapes(const lfm3_config& c) {
  std::vector<GemmShape> v;
  for (int i = 0; i < c.n_layers; ++i) {
    if (c.layer_type[i] == LFM3_LAYER_CONV) {
      v.push_back({3 * c.hidden, c.hidden, ROLE_MIXER});
      v.push_back({c.hidden, c.hidden, ROLE_MIXER});
    } else {
      v.push_back({qkvg_rows(c), c.hidden, ROLE_MIXER});
      v.push_back({c.hidden, c.n_q_heads * c.head_dim, ROLE_MIXER});
    }
    v.push_back({2 * c.ffn, c.hidden, ROLE_FFN});
    v.push_back({c.hidden, c.ffn, ROLE_FFN});
  }
  return v;
}

// Whether a linear's MFMA paths read an fp16 operand copy: always for bf16, NVFP4 and block-FP8
// (no re-tiled codes), and for affine codes at 6 bits, whose in-loop unpack is the costliest (the
// copy's 4x weight bytes cost more than the unpack saves at 4 and 8 bits, measured on the 8k
// prefill). The head never gets one for affine codes (its MFMA path dequantises in the K loop).
bool gemm_f16_copy(const LinFmt& f, int n) {
  (void)n;
  return f.fmt != FMT_AFFINE || f.bits == 6;
}

// re-tiled codes and (scale, bias) pairs (affine only) and the fp16 operand copy, each 256-byte aligned
size_t gemm_w_bytes(int n, int k, const LinFmt& f, bool f16) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t codes = f.fmt == FMT_AFFINE ? up(gemm_codes_bytes(n, k, f.bits)) + up(gemm_sb_bytes(n, k)) : 0;
  return codes + (f16 ? up(gemm_w16_bytes(n, k)) : 0);
}

Layout make_layout(const lfm3_config& c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const size_t H = c.hidden, F = c.ffn;
  const int n_conv = n_of_type(c, LFM3_LAYER_CONV), n_full = n_of_type(c, LFM3_LAYER_FULL),
            n_swa = n_of_type(c, LFM3_LAYER_SLIDING);
  L.max_rows = std::max(c.max_chunk, c.max_slots);
  L.max_pages = (c.max_ctx + kPageTokens - 1) / kPageTokens;
  L.ring_rows = c.window + c.max_chunk;
  L.max_splits = std::max(64, c.window / 64) + 1;   // attn_decode_split_keys: <= 64 full splits, window / 64 sliding
  L.big_ld = std::max<int>(3 * c.hidden, qkvg_rows(c));
  L.big_ld = (L.big_ld + 7) / 8 * 8;
  const size_t tab = (size_t)c.max_ctx * kHalfDim * 4;
  L.cos_f = take(tab); L.sin_f = take(tab); L.cos_s = take(tab); L.sin_s = take(tab);
  L.conv_slot = (size_t)n_conv * (c.conv_taps - 1) * H;
  L.conv_state = take((size_t)c.max_slots * L.conv_slot * 2);
  L.ring_layer = (size_t)c.max_slots * c.n_kv_heads * L.ring_rows * kHeadDim;
  L.ring_k = take((size_t)n_swa * L.ring_layer * 2);
  L.ring_v = take((size_t)n_swa * L.ring_layer * 2);
  L.pool_layer = (size_t)c.n_pages * c.n_kv_heads * kPageTokens * kHeadDim;
  L.pool_k = take((size_t)n_full * L.pool_layer * 2);
  L.pool_v = take((size_t)n_full * L.pool_layer * 2);
  L.page_table = take((size_t)c.max_slots * L.max_pages * 4);
  const size_t R = L.max_rows;
  L.h = take(R * H * 4);
  L.h2 = take(R * H * 4);
  L.x = take(R * H * 2);
  L.xlo = take(R * H * 2);
  L.big = take(R * L.big_ld * 4);
  L.sbuf = take(R * F * 2);
  L.mix = take(R * H * 2);
  L.qrot = take(R * c.n_q_heads * kHeadDim * 2);
  L.m = take(R * H * 4);
  L.m2 = take(R * H * 4);
  L.m3 = take((size_t)kMaxBatch * H * 4);   // decode K-split partials 3 and 4 (m2 holds partial 2)
  L.m4 = take((size_t)kMaxBatch * H * 4);
  L.xf = take(R * H * 2);
  L.part = take((size_t)c.max_slots * c.n_q_heads * L.max_splits * kPartStride * 4);
  L.keys = take((size_t)kMaxBatch * kArgmaxParts * 8);   // argmax partials [row][part]
  L.flags = take(256);                                     // device-side argument errors (bit 0: token id)
  L.vpre = take((size_t)c.max_slots * L.conv_slot * 2);
  L.vz = take((size_t)c.max_slots * n_conv * kMaxVerify * H * 2);
  L.gemm_w_bytes = 0;
  for (const auto& g : gemm_shapes(c)) {
    const LinFmt f = fmt_of(c, g.role);
    L.gemm_w_bytes += gemm_w_bytes(g.n, g.k, f, gemm_f16_copy(f, g.n));
  }
  if (c.has_embedding) {   // the tied head: codes for affine, the fp16 copy otherwise
    const LinFmt f = fmt_of(c, ROLE_EMBED);
    L.gemm_w_bytes += gemm_w_bytes(c.vocab, c.hidden, f, f.fmt != FMT_AFFINE);
  }
  L.gemm_w = take(L.gemm_w_bytes);
  L.total = off;
  return L;
}

struct LayerW {
  int type;
  int sub;  // index among layers of the same type
  const bf16_t *op_norm, *post_op, *ffn_norm, *post_ffn, *conv_kernel, *q_norm, *k_norm;
  QLinear mix_in, mix_out, w13, w2;
  GemmW g_in, g_out, g13, g2;   // their re-tiled copies for the prefill GEMM
};

}  // namespace

// Optional per-launch timing: HIP events bracket each launch of a kernel family on the context's
// stream, with the algorithmic bytes and flops that launch implies.
struct ProfRec {
  int kind;
  hipEvent_t a, b;
  double bytes, flops;
  int64_t launches;
};

struct lfm3_ctx {
  lfm3_config cfg;
  Layout L;
  hipStream_t stream;
  const uint8_t* blob;
  uint8_t* ws;
  std::vector<LayerW> layers;
  QLinear emb{};
  GemmW g_emb{};   // the head's re-tiled copy (decode batches of 3+ rows)
  const bf16_t* emb_norm = nullptr;
  std::vector<int> len;
  std::vector<int> pending;   // rows of a slot's uncommitted verify window (0: none)
  f16_t* verify_z = nullptr;  // while a verify pass runs: its slot's z rows [n_conv, kMaxVerify, H]
  std::vector<std::vector<int32_t>> pages;
  std::vector<int32_t> free_pages;
  float* capture = nullptr;
  int capture_rows = 0;
  std::string err;
  std::unordered_map<std::string, QLinear> lin_by_name;
  std::unordered_map<std::string, GemmW> gemm_by_name;
  bool prof = false;
  bool prof_open = false;    // the last record's run is still open (its end event not recorded)
  std::vector<ProfRec> prof_recs;
  std::vector<hipEvent_t> prof_pool;
  hipEvent_t ev() {
    if (prof_pool.empty()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      return e;
    }
    hipEvent_t e = prof_pool.back();
    prof_pool.pop_back();
    return e;
  }
  ~lfm3_ctx() {
    for (auto& r : prof_recs) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
    for (auto e : prof_pool) (void)hipEventDestroy(e);
  }

  template <class T> T* at(size_t off) { return (T*)(ws + off); }
  lfm3_status fail(lfm3_status s, const std::string& m) {
    err = m;
    return s;
  }
};

namespace {

// Admission of a blob: `head` holds at least the header and table (head_len bytes); blob_bytes is
// the whole blob's size, against which every tensor's byte range is checked.
bool validate_blob_impl(const lfm3_config& c, const uint8_t* head, size_t head_len, size_t blob_bytes, std::string& err,
                        std::unordered_map<std::string, Entry>* out_entries) {
  std::unordered_map<std::string, Entry> ent;
  uint64_t total = 0;
  if (!parse_header(head, head_len, ent, total, err)) return false;
  if (total != blob_bytes) { err = "blob header total " + std::to_string(total) + " != blob size " + std::to_string(blob_bytes); return false; }
  const auto exp = expected_tensors(c);
  if (ent.size() != exp.size()) {
    err = "blob holds " + std::to_string(ent.size()) + " tensors, config implies " + std::to_string(exp.size());
    return false;
  }
  for (const auto& e : exp) {
    auto it = ent.find(e.name);
    if (it == ent.end()) { err = "blob lacks tensor " + e.name; return false; }
    const Entry& en = it->second;
    if (en.dtype != e.dtype) { err = "tensor " + e.name + " has dtype " + std::to_string(en.dtype); return false; }
    if (en.ndim != e.shape.size()) { err = "tensor " + e.name + " has " + std::to_string(en.ndim) + " dims"; return false; }
    for (size_t d = 0; d < e.shape.size(); ++d)
      if (en.shape[d] != e.shape[d]) {
        err = "tensor " + e.name + " dim " + std::to_string(d) + " is " + std::to_string(en.shape[d]) + ", expected " + std::to_string(e.shape[d]);
        return false;
      }
    if (en.nbytes != elem_bytes(e)) { err = "tensor " + e.name + " byte count " + std::to_string(en.nbytes) + " != " + std::to_string(elem_bytes(e)); return false; }
    if (en.offset % 16 != 0) { err = "tensor " + e.name + " offset not 16-byte aligned"; return false; }
    if (en.offset + en.nbytes > blob_bytes) { err = "tensor " + e.name + " runs past the blob end"; return false; }
  }
  if (out_entries) *out_entries = std::move(ent);
  return true;
}

size_t blob_size_for(const lfm3_config& c) {
  const auto exp = expected_tensors(c);
  size_t off = 64 + exp.size() * 128;
  off = (off + 4095) / 4096 * 4096;
  for (const auto& e : exp) off = (off + elem_bytes(e) + 255) / 256 * 256;
  return off;
}

// Launch `fn` (returning hipError_t); when profiling, bracket it with events. A run of
// consecutive launches of one family shares one event pair: the start event goes in before the
// first launch and the end event after the last one (when a launch of another family comes, or
// when the API call ends), so no event sits between two kernels of a run. Every launch of a step
// goes through here, so a run never spans a kernel of another family.
hipError_t prof_close(lfm3_ctx* ctx) {
  if (!ctx->prof || !ctx->prof_open) return hipSuccess;
  ctx->prof_open = false;
  return hipEventRecord(ctx->prof_recs.back().b, ctx->stream);
}

template <class F>
hipError_t timed(lfm3_ctx* ctx, int kind, double bytes, double flops, F fn) {
  if (!ctx->prof) return fn();
  if (ctx->prof_open && ctx->prof_recs.back().kind == kind) {
    ProfRec& r = ctx->prof_recs.back();
    hipError_t e = fn();
    if (e != hipSuccess) return e;
    r.bytes += bytes; r.flops += flops; ++r.launches;
    return hipSuccess;
  }
  hipError_t e = prof_close(ctx);
  if (e != hipSuccess) return e;
  ProfRec r{kind, ctx->ev(), ctx->ev(), bytes, flops, 1};
  if (!r.a || !r.b) return fn();
  e = hipEventRecord(r.a, ctx->stream);
  if (e != hipSuccess) return e;
  ctx->prof_recs.push_back(r);
  ctx->prof_open = true;
  return fn();
}

// Algorithmic bytes of a weight as stored: codes (or bf16 values) and their scales.
double stored_bytes(int fmt, double n, double k, int bits, int group) {
  if (fmt == FMT_BF16) return 2.0 * n * k;
  if (fmt == FMT_NVFP4) return n * k / 2.0 + n * k / 16.0 + 8.0;
  if (fmt == FMT_FP8B) return n * k + 4.0 * std::ceil(n / 128.0) * std::ceil(k / 128.0);
  return n * (k * bits / 8.0 + 4.0 * k / group);
}
double lin_bytes(const QLinear& w) { return stored_bytes(w.fmt, w.n, w.k, w.bits, w.group); }
// the same algorithmic bytes for the weight behind a re-tiled or fp16 copy
double lin_bytes(const GemmW& w) { return stored_bytes(w.fmt, w.n, w.k, w.bits, w.group); }

#define LFM3_TRY(expr)                                                                      \
  do {                                                                                      \
    hipError_t _e = (expr);                                                                 \
    if (_e != hipSuccess) return ctx->fail(LFM3_ERR_DEVICE, std::string("HIP: ") + hipGetErrorString(_e) + " in " #expr); \
  } while (0)

KvRef kv_for(lfm3_ctx* ctx, const LayerW& lw) {
  KvRef kv{};
  const Layout& L = ctx->L;
  if (lw.type == LFM3_LAYER_FULL) {
    kv.k = ctx->at<f16_t>(L.pool_k) + (size_t)lw.sub * L.pool_layer;
    kv.v = ctx->at<f16_t>(L.pool_v) + (size_t)lw.sub * L.pool_layer;
    kv.page_table = ctx->at<int32_t>(L.page_table);
    kv.max_pages = L.max_pages;
    kv.ring = 0;
  } else {
    kv.k = ctx->at<f16_t>(L.ring_k) + (size_t)lw.sub * L.ring_layer;
    kv.v = ctx->at<f16_t>(L.ring_v) + (size_t)lw.sub * L.ring_layer;
    kv.ring = L.ring_rows;
  }
  return kv;
}

// One prefill pass (a chunk of one slot's rows, GEMM path) whose hidden input is already in h.
lfm3_status run_layers(lfm3_ctx* ctx, const Rows& rows, int capture_row0, float* hidden_out) {
  const lfm3_config& c = ctx->cfg;
  const Layout& L = ctx->L;
  hipStream_t s = ctx->stream;
  const int M = rows.n;
  const int H = c.hidden;
  float* h = ctx->at<float>(L.h);
  f16_t* x = ctx->at<f16_t>(L.x);
  float* big = ctx->at<float>(L.big);
  f16_t* sb = ctx->at<f16_t>(L.sbuf);
  f16_t* mix = ctx->at<f16_t>(L.mix);
  f16_t* qrot = ctx->at<f16_t>(L.qrot);
  float* m = ctx->at<float>(L.m);
  float* m2 = ctx->at<float>(L.m2);
  f16_t* xf = ctx->at<f16_t>(L.xf);
  f16_t* xlo = ctx->at<f16_t>(L.xlo);

  // fp32 output (STORE) or fp16 SwiGLU output
  // x_lo: the input is carried as the fp16 pair in + x_lo (two K passes over the same weight tiles;
  // the second pass is overhead, so the flops recorded stay the algorithmic 2 M N K)
  // outf2: the hidden-width outputs (mixer output projection, w2) run as two K halves, whose
  // partial sums (outf, outf2) the next residual norm adds; the narrow N would otherwise give one
  // block per CU
  auto linear = [&](const GemmW& w, const f16_t* in, int ldin, float* outf, f16_t* outb, int ldout, int epi,
                    const f16_t* x_lo = nullptr, float* outf2 = nullptr) -> hipError_t {
    const double out_bytes = epi == GEMM_SWIGLU ? (double)M * (w.n / 2) * 2.0 : (double)M * w.n * 4.0;
    const double passes = x_lo ? 2.0 : 1.0;
    const double bytes = lin_bytes(w) + passes * M * w.k * 2.0 + out_bytes;
    const double flops = 2.0 * M * (double)w.n * w.k;
    GemmArgs g{};
    g.w = w; g.x = in; g.x_lo = x_lo; g.ldx = ldin; g.m = M; g.epi = epi; g.y = outb; g.yf = outf; g.yf2 = outf2;
    g.ldy = ldout;
    return timed(ctx, LFM3_PROF_GEMM, bytes + (outf2 ? (double)M * w.n * 4.0 : 0.0), flops, [&] { return launch_gemm(s, g); });
  };
  const double norm_bytes = (double)M * H * (4 + 4 + 4 + 2);
  auto cap = [&](int layer) -> float* {
    if (!ctx->capture || layer < 0) return nullptr;
    return ctx->capture + ((size_t)layer * ctx->capture_rows + capture_row0) * H;
  };

  for (int i = 0; i < c.n_layers; ++i) {
    const LayerW& lw = ctx->layers[i];
    // h += post_ffn_norm(m) of the previous layer (if any); x = operator_norm(h)
    NormArgs na{};
    // the conv layers' operator-norm output is carried as an fp16 pair (x, x_lo) into in_proj
    na.h_in = h; na.h_out = h; na.x_out = x; na.x_lo = lw.type == LFM3_LAYER_CONV ? xlo : nullptr;
    na.rows = M; na.hidden = H; na.eps = c.norm_eps;
    na.w_pre = lw.op_norm;
    if (i > 0) { na.m = m; na.m2 = m2; na.w_post = ctx->layers[i - 1].post_ffn; na.capture = cap(i - 1); }
    LFM3_TRY(timed(ctx, LFM3_PROF_NORM, norm_bytes, 0, [&] { return launch_resid_norm(s, na); }));

    if (lw.type == LFM3_LAYER_CONV) {
      LFM3_TRY(linear(lw.g_in, x, H, big, nullptr, L.big_ld, GEMM_STORE, xlo));
      ConvArgs ca{};
      ca.bcx = big; ca.ld = L.big_ld; ca.kernel = lw.conv_kernel;
      ca.state = ctx->at<f16_t>(L.conv_state) + (size_t)lw.sub * (c.conv_taps - 1) * H;
      ca.slot_stride = (int64_t)L.conv_slot;
      ca.out = mix; ca.rows = rows; ca.hidden = H; ca.taps = c.conv_taps;
      ca.z_out = ctx->verify_z ? ctx->verify_z + (size_t)lw.sub * kMaxVerify * H : nullptr;
      LFM3_TRY(timed(ctx, LFM3_PROF_CONV, (double)M * H * (12 + 2) + 2.0 * H * 2 * (c.conv_taps - 1), 0,
                     [&] { return launch_conv(s, ca); }));
    } else {
      LFM3_TRY(linear(lw.g_in, x, H, big, nullptr, L.big_ld, GEMM_STORE));
      const bool full = lw.type == LFM3_LAYER_FULL;
      QkRopeArgs qa{};
      qa.qkvg = big; qa.ld = L.big_ld; qa.q_norm = lw.q_norm; qa.k_norm = lw.k_norm;
      qa.cos_t = ctx->at<float>(full ? L.cos_f : L.cos_s);
      qa.sin_t = ctx->at<float>(full ? L.sin_f : L.sin_s);
      qa.q_out = qrot; qa.kv = kv_for(ctx, lw); qa.rows = rows;
      qa.n_q_heads = c.n_q_heads; qa.n_kv_heads = c.n_kv_heads; qa.eps = c.norm_eps;
      LFM3_TRY(timed(ctx, LFM3_PROF_OTHER, (double)M * L.big_ld * 4, 0, [&] { return launch_qk_rope(s, qa); }));
      AttnArgs aa{};
      aa.q = qrot;
      aa.gate = big + (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * kHeadDim;
      aa.ldg = L.big_ld; aa.kv = qa.kv; aa.rows = rows;
      aa.window = full ? 0 : c.window;
      aa.n_q_heads = c.n_q_heads; aa.n_kv_heads = c.n_kv_heads; aa.out = mix;
      aa.part = ctx->at<float>(L.part);
      {
        double fl = 0;
        for (int r = 0; r < M; ++r) {
          const double p = rows.pos0 + r;
          const double t = full ? p + 1 : std::min(p + 1, (double)c.window);
          fl += 4.0 * kHeadDim * c.n_q_heads * t;
        }
        LFM3_TRY(timed(ctx, LFM3_PROF_ATTN_PREFILL, 0, fl, [&] { return launch_attn_prefill(s, aa); }));
      }
    }
    LFM3_TRY(linear(lw.g_out, mix, H, m, nullptr, H, GEMM_STORE, nullptr, m2));
    // h += post_operator_norm(m); x = ffn_norm(h)
    NormArgs nb{};
    nb.h_in = h; nb.h_out = h; nb.x_out = x; nb.rows = M; nb.hidden = H; nb.eps = c.norm_eps;
    nb.m = m; nb.m2 = m2; nb.w_post = lw.post_op; nb.w_pre = lw.ffn_norm;
    LFM3_TRY(timed(ctx, LFM3_PROF_NORM, norm_bytes + (double)M * H * 4, 0, [&] { return launch_resid_norm(s, nb); }));
    LFM3_TRY(linear(lw.g13, x, H, nullptr, sb, c.ffn, GEMM_SWIGLU));
    LFM3_TRY(linear(lw.g2, sb, c.ffn, m, nullptr, H, GEMM_STORE, nullptr, m2));
  }
  NormArgs nf{};
  nf.h_in = h; nf.h_out = h; nf.x_out = xf; nf.rows = M; nf.hidden = H; nf.eps = c.norm_eps;
  nf.m = m; nf.m2 = m2; nf.w_post = ctx->layers[c.n_layers - 1].post_ffn; nf.w_pre = ctx->emb_norm;
  nf.capture = cap(c.n_layers - 1);
  nf.x_copy = hidden_out;
  LFM3_TRY(timed(ctx, LFM3_PROF_NORM, norm_bytes, 0, [&] { return launch_resid_norm(s, nf); }));
  return LFM3_OK;
}

// One decode step: one row per slot, h input already in the first residual buffer. GEMVs take
// their RMSNorm'd input through the fused prologue for batches of at most 2 rows (each block
// recomputes the norm from L2-resident rows); larger batches run the norm once and feed plain
// GEMVs. Both use the same arithmetic. Ends with the tied head and the argmax when asked.
lfm3_status run_decode(lfm3_ctx* ctx, const Rows& rows, float* hidden_out, float* logits, int32_t* ids) {
  const lfm3_config& c = ctx->cfg;
  const Layout& L = ctx->L;
  hipStream_t s = ctx->stream;
  const int M = rows.n;
  const int H = c.hidden;
  float* cur = ctx->at<float>(L.h);
  float* oth = ctx->at<float>(L.h2);
  f16_t* x = ctx->at<f16_t>(L.x);
  float* big = ctx->at<float>(L.big);
  f16_t* sb = ctx->at<f16_t>(L.sbuf);
  f16_t* mix = ctx->at<f16_t>(L.mix);
  float* m = ctx->at<float>(L.m);
  // the mixer / FFN output projections of 3+ rows split K in four (sgemm_store_ksplit); m then
  // holds the first quarter's sums and mq[0..2] the others, which the next norm adds
  float* mq[3] = {ctx->at<float>(L.m2), ctx->at<float>(L.m3), ctx->at<float>(L.m4)};
  bool m_split = false;
  f16_t* xf = ctx->at<f16_t>(L.xf);
  f16_t* xlo = ctx->at<f16_t>(L.xlo);
  const bool fuse = M <= 2;
  auto cap = [&](int layer) -> float* {
    if (!ctx->capture || layer < 0) return nullptr;
    return ctx->capture + (size_t)layer * ctx->capture_rows * H;
  };
  auto gemv_bytes = [&](const QLinear& w, double out_bytes) { return lin_bytes(w) + (double)M * w.k * 2.0 + out_bytes; };
  // batches of 3 rows and more run the layers' linears on MFMA from the re-tiled weights (one read
  // of the weights for all rows); 1 and 2 rows keep the exact GEMV with its fused norm prologue
  const bool mfma = M >= 3;
  auto gemv = [&](GemvArgs& g, double out_bytes, const GemmW* gw = nullptr) -> hipError_t {
    const double fl = 2.0 * M * (double)g.w.n * g.w.k;
    if (mfma && gw && (g.x_lo ? 2 * M : M) <= 64)
      return timed(ctx, LFM3_PROF_GEMV, gemv_bytes(g.w, out_bytes), fl, [&] { return launch_sgemm(s, *gw, g); });
    if (mfma && gw && g.x_lo && g.epi == GEMV_STORE && !g.yf_part[0]) {
      // an input carried as a pair past 32 rows (more than the MFMA kernel's 64 operand rows): one
      // launch per 32 rows; a row's sums do not depend on the rows that share its launch
      for (int r0 = 0; r0 < M; r0 += 32) {
        GemvArgs gp = g;
        gp.batch = std::min(32, M - r0);
        gp.x = g.x + (size_t)r0 * g.ldx;
        gp.x_lo = g.x_lo + (size_t)r0 * g.ldx;
        gp.yf = g.yf + (size_t)r0 * g.ldy;
        const double part = (double)gp.batch / M;
        const hipError_t e = timed(ctx, LFM3_PROF_GEMV, gemv_bytes(g.w, out_bytes) * part, fl * part,
                                   [&] { return launch_sgemm(s, *gw, gp); });
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
    return timed(ctx, LFM3_PROF_GEMV, gemv_bytes(g.w, out_bytes), fl, [&] { return launch_gemv(s, g); });
  };
  // GEMV whose input is rmsnorm(cur [+ rmsnorm(m) * w_post]) * w_pre
  // split: the normed input is carried as the fp16 pair x + x_lo (the conv layers' operator-norm
  // output, which feeds in_proj); a fused split prologue handles one row
  auto normed_gemv = [&](GemvArgs& g, const bf16_t* w_post, const bf16_t* w_pre, float* capture, float* x_copy,
                         double out_bytes, bool split = false, const GemmW* gw = nullptr) -> hipError_t {
    g.batch = M;
    if (fuse && (!split || M == 1)) {
      g.h_src = cur; g.m = w_post ? m : nullptr; g.w_post = w_post; g.w_pre = w_pre; g.eps = c.norm_eps;
      g.h_dst = oth; g.capture = capture; g.capture_ld = H; g.x_copy = x_copy; g.split_x = split;
      hipError_t e = gemv(g, out_bytes + (split ? (double)M * H * 2 : 0.0));
      if (w_post) std::swap(cur, oth);
      return e;
    }
    NormArgs na{};
    na.h_in = cur; na.h_out = cur; na.m = w_post ? m : nullptr; na.w_post = w_post; na.w_pre = w_pre;
    if (w_post && m_split) { na.m2 = mq[0]; na.m3 = mq[1]; na.m4 = mq[2]; }
    na.x_out = x; na.x_lo = split ? xlo : nullptr;
    na.capture = capture; na.x_copy = x_copy; na.rows = M; na.hidden = H; na.eps = c.norm_eps;
    hipError_t e = timed(ctx, LFM3_PROF_NORM, (double)M * H * 14, 0, [&] { return launch_resid_norm(s, na); });
    if (e != hipSuccess) return e;
    g.x = x; g.x_lo = na.x_lo; g.ldx = H;
    return gemv(g, out_bytes + (split ? (double)M * H * 2 : 0.0), gw);
  };

  for (int i = 0; i < c.n_layers; ++i) {
    const LayerW& lw = ctx->layers[i];
    const bf16_t* w_post = i > 0 ? ctx->layers[i - 1].post_ffn : nullptr;
    // sliding layers at 1-2 rows: the o_proj GEMV merges the attention's split partials itself
    // (a window of at most kFusedMergeSplits tiles), which saves the merge launch
    GemvArgs merge_in{};
    if (lw.type == LFM3_LAYER_CONV && mfma) {
      // 3+ rows: in_proj as a plain MFMA linear over every CU (one block per 32-row tile of
      // B | C | x; past 32 rows one launch per 32 rows), then the gated conv with each row's kept
      // state in its own small launch
      GemvArgs g{};
      g.w = lw.mix_in; g.epi = GEMV_STORE; g.yf = big; g.ldy = L.big_ld;
      LFM3_TRY(normed_gemv(g, w_post, lw.op_norm, cap(i - 1), nullptr, (double)M * lw.mix_in.n * 4, true, &lw.g_in));
      ConvArgs ca{};
      ca.bcx = big; ca.ld = L.big_ld; ca.kernel = lw.conv_kernel;
      ca.state = ctx->at<f16_t>(L.conv_state) + (size_t)lw.sub * (c.conv_taps - 1) * H;
      ca.slot_stride = (int64_t)L.conv_slot;
      ca.out = mix; ca.rows = rows; ca.hidden = H; ca.taps = c.conv_taps;
      LFM3_TRY(timed(ctx, LFM3_PROF_CONV, (double)M * H * (12 + 2 + 4 * (c.conv_taps - 1)), 0,
                     [&] { return launch_conv(s, ca); }));
    } else if (lw.type == LFM3_LAYER_CONV) {
      GemvArgs g{};
      g.w = lw.mix_in; g.epi = GEMV_CONV; g.y = mix; g.ldy = H;
      g.conv_kernel = lw.conv_kernel;
      g.conv_state = ctx->at<f16_t>(L.conv_state) + (size_t)lw.sub * (c.conv_taps - 1) * H;
      g.conv_slot_stride = (int64_t)L.conv_slot;
      g.conv_taps = c.conv_taps;
      for (int b = 0; b < M; ++b) g.conv_slot[b] = rows.slot[b];
      // 1-2 rows: the exact GEMV with the fused norm prologue and the conv epilogue
      LFM3_TRY(normed_gemv(g, w_post, lw.op_norm, cap(i - 1), nullptr, (double)M * H * (2 + 4 * (c.conv_taps - 1)), true));
    } else {
      GemvArgs g{};
      g.w = lw.mix_in; g.epi = GEMV_STORE; g.yf = big; g.ldy = L.big_ld;
      LFM3_TRY(normed_gemv(g, w_post, lw.op_norm, cap(i - 1), nullptr, (double)M * lw.mix_in.n * 4, false, &lw.g_in));
      const bool full = lw.type == LFM3_LAYER_FULL;
      AttnDecodeArgs aa{};
      aa.qkvg = big; aa.ld = L.big_ld; aa.gate_col = (c.n_q_heads + 2 * c.n_kv_heads) * kHeadDim;
      aa.q_norm = lw.q_norm; aa.k_norm = lw.k_norm;
      aa.cos_t = ctx->at<float>(full ? L.cos_f : L.cos_s);
      aa.sin_t = ctx->at<float>(full ? L.sin_f : L.sin_s);
      aa.kv = kv_for(ctx, lw); aa.rows = rows;
      aa.window = full ? 0 : c.window;
      aa.n_q_heads = c.n_q_heads; aa.n_kv_heads = c.n_kv_heads; aa.eps = c.norm_eps;
      aa.out = mix; aa.part = ctx->at<float>(L.part);
      int ms = 1;
      double kv_bytes = 0;
      for (int r = 0; r < M; ++r) {
        const int lo = full ? 0 : std::max(0, rows.pos[r] - (c.window - 1));
        const int ns = (rows.pos[r] - lo) / attn_decode_split_keys(!full, rows.pos[r] - lo + 1) + 1;
        ms = std::max(ms, ns);
        merge_in.merge_splits[r] = ns;
        kv_bytes += (double)(rows.pos[r] - lo + 1) * c.n_kv_heads * kHeadDim * 2 * 2;
      }
      aa.max_splits = ms;
      if (!mfma && !full && c.window <= kFusedMergeSplits * 64) {
        aa.merge_in_consumer = 1;
        merge_in.part = aa.part; merge_in.part_splits = ms;
        merge_in.gate_src = big + aa.gate_col; merge_in.gate_ld = L.big_ld;
      }
      LFM3_TRY(timed(ctx, LFM3_PROF_ATTN_DECODE, kv_bytes, 0, [&] { return launch_attn_decode(s, aa); }));
    }
    {
      GemvArgs g = merge_in;
      g.w = lw.mix_out; g.x = mix; g.ldx = H; g.batch = M; g.epi = GEMV_STORE; g.yf = m; g.ldy = H;
      if (mfma) for (int q = 0; q < 3; ++q) g.yf_part[q] = mq[q];
      LFM3_TRY(gemv(g, (double)M * H * 4, &lw.g_out));
      m_split = mfma && sgemm_store_ksplit(lw.g_out);
    }
    {
      GemvArgs g{};
      g.w = lw.w13; g.epi = GEMV_SWIGLU; g.y = sb; g.ldy = c.ffn;
      LFM3_TRY(normed_gemv(g, lw.post_op, lw.ffn_norm, nullptr, nullptr, (double)M * c.ffn * 2, false, &lw.g13));
    }
    {
      GemvArgs g{};
      g.w = lw.w2; g.x = sb; g.ldx = c.ffn; g.batch = M; g.epi = GEMV_STORE; g.yf = m; g.ldy = H;
      if (mfma) for (int q = 0; q < 3; ++q) g.yf_part[q] = mq[q];
      LFM3_TRY(gemv(g, (double)M * H * 4, &lw.g2));
      m_split = mfma && sgemm_store_ksplit(lw.g2);
    }
  }
  const bf16_t* last_post = ctx->layers[c.n_layers - 1].post_ffn;
  if (c.has_embedding && (logits || ids)) {
    GemvArgs g{};
    g.w = ctx->emb; g.epi = GEMV_LOGITS; g.logits = logits; g.ld_logits = c.vocab;
    g.keys = ctx->at<uint64_t>(L.keys);
    LFM3_TRY(normed_gemv(g, last_post, ctx->emb_norm, cap(c.n_layers - 1), hidden_out, logits ? (double)M * c.vocab * 4 : 0.0,
                         false, &ctx->g_emb));
    LFM3_TRY(timed(ctx, LFM3_PROF_OTHER, (16.0 * kArgmaxParts + 4) * M, 0, [&] { return launch_argmax_finalize(s, g.keys, ids, M); }));
  } else {
    NormArgs nf{};
    nf.h_in = cur; nf.h_out = cur; nf.x_out = xf; nf.rows = M; nf.hidden = H; nf.eps = c.norm_eps;
    nf.m = m; nf.w_post = last_post; nf.w_pre = ctx->emb_norm;
    if (m_split) { nf.m2 = mq[0]; nf.m3 = mq[1]; nf.m4 = mq[2]; }
    nf.capture = cap(c.n_layers - 1);
    nf.x_copy = hidden_out;
    LFM3_TRY(timed(ctx, LFM3_PROF_NORM, (double)M * H * 14, 0, [&] { return launch_resid_norm(s, nf); }));
  }
  return LFM3_OK;
}

lfm3_status head(lfm3_ctx* ctx, const f16_t* xrows, int n, float* logits, int32_t* ids) {
  if (!logits && !ids) return LFM3_OK;
  GemvArgs g{};
  g.w = ctx->emb; g.x = xrows; g.ldx = ctx->cfg.hidden; g.batch = n; g.epi = GEMV_LOGITS;
  g.logits = logits; g.ld_logits = ctx->cfg.vocab; g.keys = ctx->at<uint64_t>(ctx->L.keys);
  const double bytes = lin_bytes(g.w) + (double)n * g.w.k * 2 + (logits ? (double)n * g.w.n * 4 : 0.0);
  LFM3_TRY(timed(ctx, LFM3_PROF_GEMV, bytes, 2.0 * n * g.w.n * g.w.k, [&] { return launch_gemv(ctx->stream, g); }));
  LFM3_TRY(timed(ctx, LFM3_PROF_OTHER, (16.0 * kArgmaxParts + 4) * n, 0, [&] { return launch_argmax_finalize(ctx->stream, g.keys, ids, n); }));
  return LFM3_OK;
}

// Reserve pages so `slot` can hold `new_len` positions; only host state changes here, the
// page-table writes are returned in `writes` (index, page) to be enqueued by the caller.
bool reserve_pages(lfm3_ctx* ctx, int slot, int new_len, std::vector<std::pair<int, int>>& writes, int& budget) {
  if (n_of_type(ctx->cfg, LFM3_LAYER_FULL) == 0) return true;
  const int need = (new_len + kPageTokens - 1) / kPageTokens;
  const int have = (int)ctx->pages[slot].size();
  if (need - have > budget) return false;
  budget -= std::max(0, need - have);
  (void)writes;
  return true;
}

lfm3_status commit_pages(lfm3_ctx* ctx, int slot, int new_len) {
  if (n_of_type(ctx->cfg, LFM3_LAYER_FULL) == 0) return LFM3_OK;
  const int need = (new_len + kPageTokens - 1) / kPageTokens;
  auto& pg = ctx->pages[slot];
  const int first = (int)pg.size();
  while ((int)pg.size() < need) {
    pg.push_back(ctx->free_pages.back());
    ctx->free_pages.pop_back();
  }
  if ((int)pg.size() > first) {
    LFM3_TRY(timed(ctx, LFM3_PROF_OTHER, 8.0 * (need - first), 0, [&] { return launch_set_pages(ctx->stream, ctx->at<int32_t>(ctx->L.page_table), slot * ctx->L.max_pages + first,
                              (int)pg.size() - first, pg.data() + first); }));
  }
  return LFM3_OK;
}

// A kept state of a slot at `length` positions, in a caller buffer: the conv states of every conv
// layer, the full layers' keys and values of positions [0, length) and the sliding layers' of the
// last window - 1 positions (all the next position sees), each region 256-byte aligned.
struct StateLayout {
  size_t conv, full, swa, total;
  int swa_p0, swa_n;
  size_t row;   // bytes of one position's keys (or values): n_kv * 128 fp16
};

StateLayout state_layout(const lfm3_config& c, const Layout& L, int length) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  StateLayout s{};
  s.row = (size_t)c.n_kv_heads * kHeadDim * 2;
  s.swa_n = std::min(length, c.window - 1);
  s.swa_p0 = length - s.swa_n;
  s.conv = 0;
  s.full = up(L.conv_slot * 2);
  s.swa = s.full + up((size_t)n_of_type(c, LFM3_LAYER_FULL) * 2 * length * s.row);
  s.total = s.swa + up((size_t)n_of_type(c, LFM3_LAYER_SLIDING) * 2 * s.swa_n * s.row);
  return s;
}

// Move a slot's state between the cache and a state buffer (dir 0: save, 1: load); the slot's
// pages for `length` positions are in its page table already.
lfm3_status move_state(lfm3_ctx* ctx, int slot, int length, uint8_t* buf, int dir) {
  const lfm3_config& c = ctx->cfg;
  const Layout& L = ctx->L;
  const StateLayout sl = state_layout(c, L, length);
  f16_t* conv = ctx->at<f16_t>(L.conv_state) + (size_t)slot * L.conv_slot;
  if (L.conv_slot) {
    if (dir == 0) LFM3_TRY(launch_copy(ctx->stream, buf + sl.conv, conv, L.conv_slot * 2));
    else LFM3_TRY(launch_copy(ctx->stream, conv, buf + sl.conv, L.conv_slot * 2));
  }
  for (const LayerW& lw : ctx->layers) {
    if (lw.type == LFM3_LAYER_CONV) continue;
    const KvRef kv = kv_for(ctx, lw);
    const bool full = lw.type == LFM3_LAYER_FULL;
    const int p0 = full ? 0 : sl.swa_p0, n = full ? length : sl.swa_n;
    uint8_t* k = buf + (full ? sl.full : sl.swa) + (size_t)lw.sub * 2 * n * sl.row;
    uint8_t* v = k + (size_t)n * sl.row;
    LFM3_TRY(launch_kv_move(ctx->stream, kv, slot, p0, n, (f16_t*)k, (f16_t*)v, c.n_kv_heads, dir));
  }
  return LFM3_OK;
}

}  // namespace

// ================================================================================================
// C ABI
// ================================================================================================
extern "C" {

lfm3_status lfm3_query_sizes(const lfm3_config* cfg, size_t* blob_bytes, size_t* workspace_bytes) {
  if (!cfg) { g_err = "cfg is NULL"; return LFM3_ERR_ARG; }
  std::string err;
  if (!check_config(*cfg, err)) { g_err = err; return LFM3_ERR_CONFIG; }
  if (blob_bytes) *blob_bytes = blob_size_for(*cfg);
  if (workspace_bytes) *workspace_bytes = make_layout(*cfg).total;
  return LFM3_OK;
}

lfm3_status lfm3_validate_blob(const lfm3_config* cfg, const void* blob_host, size_t blob_bytes, char* err, size_t err_len) {
  std::string e;
  lfm3_status st = LFM3_OK;
  if (!cfg || !blob_host) { e = "cfg or blob is NULL"; st = LFM3_ERR_ARG; }
  else if (!check_config(*cfg, e)) st = LFM3_ERR_CONFIG;
  else if (!validate_blob_impl(*cfg, (const uint8_t*)blob_host, blob_bytes, blob_bytes, e, nullptr)) st = LFM3_ERR_BLOB;
  if (st != LFM3_OK) {
    g_err = e;
    if (err && err_len) { strncpy(err, e.c_str(), err_len - 1); err[err_len - 1] = 0; }
  }
  return st;
}

lfm3_status lfm3_create(const lfm3_config* cfg, const void* blob_dev, size_t blob_bytes, void* workspace_dev,
                        size_t workspace_bytes, void* hip_stream, lfm3_ctx** out) {
  if (!cfg || !blob_dev || !workspace_dev || !out) { g_err = "NULL argument to lfm3_create"; return LFM3_ERR_ARG; }
  *out = nullptr;
  std::string err;
  if (!check_config(*cfg, err)) { g_err = err; return LFM3_ERR_CONFIG; }
  const Layout L = make_layout(*cfg);
  if (workspace_bytes < L.total) {
    g_err = "workspace " + std::to_string(workspace_bytes) + " B < required " + std::to_string(L.total) + " B";
    return LFM3_ERR_CAPACITY;
  }
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) { g_err = "no HIP device"; return LFM3_ERR_DEVICE; }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) { g_err = std::string("device is ") + prop.gcnArchName + ", this build runs gfx950"; return LFM3_ERR_DEVICE; }
  // read the header back for admission
  uint64_t hdr[5];
  if (blob_bytes < 64 || hipMemcpy(hdr, blob_dev, 40, hipMemcpyDeviceToHost) != hipSuccess) { g_err = "cannot read the blob header"; return LFM3_ERR_BLOB; }
  uint64_t data_off = hdr[3];
  if (data_off > blob_bytes || data_off < 64) { g_err = "blob data offset out of range"; return LFM3_ERR_BLOB; }
  std::vector<uint8_t> head(data_off);
  if (hipMemcpy(head.data(), blob_dev, data_off, hipMemcpyDeviceToHost) != hipSuccess) { g_err = "cannot read the blob table"; return LFM3_ERR_BLOB; }
  std::unordered_map<std::string, Entry> ent;
  if (!validate_blob_impl(*cfg, head.data(), head.size(), blob_bytes, err, &ent)) { g_err = err; return LFM3_ERR_BLOB; }
  auto* ctx = new lfm3_ctx();
  ctx->cfg = *cfg;
  ctx->L = L;
  ctx->stream = (hipStream_t)hip_stream;
  ctx->blob = (const uint8_t*)blob_dev;
  ctx->ws = (uint8_t*)workspace_dev;
  const lfm3_config& c = *cfg;
  auto bf = [&](const std::string& n) { return (const bf16_t*)(ctx->blob + ent.at(n).offset); };
  bool scales_ok = true;
  auto lin = [&](const std::string& n, int N, int K, const LinFmt& f) {
    QLinear q{};
    q.n = N; q.k = K; q.bits = f.bits; q.group = f.group; q.fmt = f.fmt; q.tscale = 1.f;
    if (f.fmt == FMT_AFFINE) {
      q.q = ctx->blob + ent.at(n + ".q").offset;
      q.scales = bf(n + ".scales");
      q.biases = bf(n + ".biases");
    } else if (f.fmt == FMT_BF16) {
      q.q = ctx->blob + ent.at(n + ".weight").offset;
    } else if (f.fmt == FMT_NVFP4) {
      q.q = ctx->blob + ent.at(n + ".fp4").offset;
      q.bscale = ctx->blob + ent.at(n + ".block_scales").offset;
      // the tensor scale is applied; the static input scale is admitted but not applied (the
      // weights are used weight-only: activations keep their own precision)
      float ts = 0.f;
      if (hipMemcpy(&ts, ctx->blob + ent.at(n + ".tensor_scale").offset, 4, hipMemcpyDeviceToHost) != hipSuccess ||
          !(ts > 0.f) || !std::isfinite(ts))
        scales_ok = false;
      q.tscale = ts;
    } else {
      q.q = ctx->blob + ent.at(n + ".fp8").offset;
      q.bscale = ctx->blob + ent.at(n + ".block_scales").offset;
    }
    ctx->lin_by_name[n] = q;
    return q;
  };
  const LinFmt fm = fmt_of(c, ROLE_MIXER), ff = fmt_of(c, ROLE_FFN);
  int sub[3] = {0, 0, 0};
  for (int i = 0; i < c.n_layers; ++i) {
    const std::string p = "layers." + std::to_string(i) + ".";
    LayerW lw{};
    lw.type = c.layer_type[i];
    lw.sub = sub[lw.type]++;
    lw.op_norm = bf(p + "operator_norm");
    lw.post_op = bf(p + "post_operator_norm");
    lw.ffn_norm = bf(p + "ffn_norm");
    lw.post_ffn = bf(p + "post_ffn_norm");
    if (lw.type == LFM3_LAYER_CONV) {
      lw.conv_kernel = bf(p + "conv.kernel");
      lw.mix_in = lin(p + "conv.in_proj", 3 * c.hidden, c.hidden, fm);
      lw.mix_out = lin(p + "conv.out_proj", c.hidden, c.hidden, fm);
    } else {
      lw.q_norm = bf(p + "attn.q_norm");
      lw.k_norm = bf(p + "attn.k_norm");
      lw.mix_in = lin(p + "attn.qkvg_proj", qkvg_rows(c), c.hidden, fm);
      lw.mix_out = lin(p + "attn.o_proj", c.hidden, c.n_q_heads * c.head_dim, fm);
    }
    lw.w13 = lin(p + "ffn.w13", 2 * c.ffn, c.hidden, ff);
    lw.w2 = lin(p + "ffn.w2", c.hidden, c.ffn, ff);
    ctx->layers.push_back(lw);
  }
  if (c.has_embedding) ctx->emb = lin("embedding", c.vocab, c.hidden, fmt_of(c, ROLE_EMBED));
  if (!scales_ok) {
    delete ctx;
    g_err = "an NVFP4 tensor scale is not a finite positive number (or cannot be read)";
    return LFM3_ERR_BLOB;
  }
  ctx->emb_norm = bf("embedding_norm");

  // re-tiled copies of the prefill GEMM weights, in the order gemm_shapes lists them
  {
    size_t goff = L.gemm_w;
    hipError_t e = hipSuccess;
    // with16: also the fp16 operand copy the MFMA paths read (affine: from the re-tiled codes with
    // the GEMM's own dequantisation; other formats: straight from the stored weight, which then has
    // no re-tiled codes)
    auto retile = [&](const QLinear& q, const std::string& name, bool with16) {
      GemmW g{};
      auto up = [](size_t b) { return (b + 255) / 256 * 256; };
      const bool affine = q.fmt == FMT_AFFINE;
      uint8_t* base = ctx->at<uint8_t>(goff);
      uint8_t* codes = affine ? base : nullptr;
      uint32_t* sbp = affine ? (uint32_t*)(codes + up(gemm_codes_bytes(q.n, q.k, q.bits))) : nullptr;
      uint32_t* w16 = with16 ? (affine ? (uint32_t*)((uint8_t*)sbp + up(gemm_sb_bytes(q.n, q.k))) : (uint32_t*)base) : nullptr;
      goff += gemm_w_bytes(q.n, q.k, LinFmt{q.fmt, q.bits, q.group}, with16);
      g.codes = codes; g.sb = sbp; g.n = q.n; g.k = q.k; g.bits = q.bits; g.group = q.group; g.ntile = (q.n + 31) / 32;
      g.fmt = q.fmt;
      if (affine) {
        if (e == hipSuccess) e = launch_repack_gemm(ctx->stream, q, codes, sbp);
        if (with16 && e == hipSuccess) e = launch_repack_gemm16(ctx->stream, g, w16);
      } else if (e == hipSuccess) {
        e = launch_make_w16(ctx->stream, q, w16);
      }
      g.w16 = w16;
      ctx->gemm_by_name[name] = g;
      return g;
    };
    for (int i = 0; i < c.n_layers; ++i) {
      LayerW& lw = ctx->layers[i];
      const std::string p = "layers." + std::to_string(i) + ".";
      const bool conv = lw.type == LFM3_LAYER_CONV;
      lw.g_in = retile(lw.mix_in, p + (conv ? "conv.in_proj" : "attn.qkvg_proj"), gemm_f16_copy(fm, lw.mix_in.n));
      lw.g_out = retile(lw.mix_out, p + (conv ? "conv.out_proj" : "attn.o_proj"), gemm_f16_copy(fm, lw.mix_out.n));
      lw.g13 = retile(lw.w13, p + "ffn.w13", gemm_f16_copy(ff, lw.w13.n));
      lw.g2 = retile(lw.w2, p + "ffn.w2", gemm_f16_copy(ff, lw.w2.n));
    }
    if (c.has_embedding) {
      ctx->g_emb = retile(ctx->emb, "embedding", ctx->emb.fmt != FMT_AFFINE);
      ctx->gemm_by_name.erase("embedding");   // the GEMM hook paths stay off the head
    }
    if (e != hipSuccess || goff != L.gemm_w + L.gemm_w_bytes) {
      delete ctx;
      g_err = e != hipSuccess ? std::string("GEMM weight re-tiling failed: ") + hipGetErrorString(e) : "GEMM weight layout mismatch";
      return LFM3_ERR_DEVICE;
    }
  }
  ctx->len.assign(c.max_slots, 0);
  ctx->pending.assign(c.max_slots, 0);
  ctx->pages.assign(c.max_slots, {});
  for (int p = c.n_pages - 1; p >= 0; --p) ctx->free_pages.push_back(p);

  // RoPE tables: angle p * theta^(-2i/head_dim) in float64, stored fp32; pairs past n_pairs get
  // angle 0 (cos 1, sin 0).
  {
    const size_t n = (size_t)c.max_ctx * kHalfDim;
    std::vector<float> cf(n), sf(n), cs(n), ss(n);
    for (int i = 0; i < kHalfDim; ++i) {
      const double invf = i < c.rope_pairs_full ? std::pow(c.rope_theta_full, -2.0 * i / c.head_dim) : 0.0;
      const double invs = i < c.rope_pairs_sliding ? std::pow(c.rope_theta_sliding, -2.0 * i / c.head_dim) : 0.0;
      for (int p = 0; p < c.max_ctx; ++p) {
        const double af = (double)p * invf, as = (double)p * invs;
        cf[(size_t)p * kHalfDim + i] = (float)std::cos(af);
        sf[(size_t)p * kHalfDim + i] = (float)std::sin(af);
        cs[(size_t)p * kHalfDim + i] = (float)std::cos(as);
        ss[(size_t)p * kHalfDim + i] = (float)std::sin(as);
      }
    }
    bool ok = hipMemcpy(ctx->at<float>(L.cos_f), cf.data(), n * 4, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(ctx->at<float>(L.sin_f), sf.data(), n * 4, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(ctx->at<float>(L.cos_s), cs.data(), n * 4, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(ctx->at<float>(L.sin_s), ss.data(), n * 4, hipMemcpyHostToDevice) == hipSuccess;
    if (!ok) { delete ctx; g_err = "RoPE table upload failed"; return LFM3_ERR_DEVICE; }
  }
  // zero the conv states, page table and argmax keys
  if (launch_zero(ctx->stream, ctx->at<void>(L.conv_state), (size_t)c.max_slots * L.conv_slot * 2) != hipSuccess ||
      launch_zero(ctx->stream, ctx->at<void>(L.page_table), (size_t)c.max_slots * L.max_pages * 4) != hipSuccess ||
      launch_zero(ctx->stream, ctx->at<void>(L.keys), (size_t)kMaxBatch * kArgmaxParts * 8) != hipSuccess ||
      launch_zero(ctx->stream, ctx->at<void>(L.flags), 256) != hipSuccess) {
    delete ctx;
    g_err = "workspace clear failed";
    return LFM3_ERR_DEVICE;
  }
  *out = ctx;
  return LFM3_OK;
}

void lfm3_destroy(lfm3_ctx* ctx) { delete ctx; }

lfm3_status lfm3_prefill(lfm3_ctx* ctx, int32_t slot, const int32_t* tokens_dev, const uint16_t* hidden_dev, int32_t n_rows,
                         float* logits_last_dev, int32_t* argmax_last_dev, float* hidden_out_dev) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  const lfm3_config& c = ctx->cfg;
  if (slot < 0 || slot >= c.max_slots) return ctx->fail(LFM3_ERR_SLOT, "slot " + std::to_string(slot) + " outside [0, max_slots)");
  if (n_rows < 1) return ctx->fail(LFM3_ERR_ARG, "n_rows must be >= 1");
  if ((tokens_dev == nullptr) == (hidden_dev == nullptr)) return ctx->fail(LFM3_ERR_ARG, "pass exactly one of tokens and hidden");
  if (tokens_dev && !c.has_embedding) return ctx->fail(LFM3_ERR_ARG, "token input needs has_embedding = 1");
  if ((logits_last_dev || argmax_last_dev) && !c.has_embedding) return ctx->fail(LFM3_ERR_ARG, "logits need the tied head (has_embedding = 1)");
  if (ctx->pending[slot]) return ctx->fail(LFM3_ERR_ARG, "slot " + std::to_string(slot) + " has an uncommitted verify window");
  if ((int64_t)ctx->len[slot] + n_rows > c.max_ctx)
    return ctx->fail(LFM3_ERR_CAPACITY, "slot length " + std::to_string(ctx->len[slot]) + " + rows " + std::to_string(n_rows) + " > max_ctx");
  if (ctx->capture && n_rows > ctx->capture_rows) return ctx->fail(LFM3_ERR_CAPACITY, "capture buffer holds fewer rows than this call");
  std::vector<std::pair<int, int>> writes;
  int budget = (int)ctx->free_pages.size();
  if (!reserve_pages(ctx, slot, ctx->len[slot] + n_rows, writes, budget)) return ctx->fail(LFM3_ERR_CAPACITY, "KV page pool exhausted");
  lfm3_status st = commit_pages(ctx, slot, ctx->len[slot] + n_rows);
  if (st != LFM3_OK) return st;
  const int H = c.hidden;
  float* h = ctx->at<float>(ctx->L.h);
  for (int r0 = 0; r0 < n_rows; r0 += c.max_chunk) {
    const int M = std::min(c.max_chunk, n_rows - r0);
    Rows rows{};
    rows.n = M; rows.mode = 0; rows.slot0 = slot; rows.pos0 = ctx->len[slot];
    if (tokens_dev) {
      LFM3_TRY(timed(ctx, LFM3_PROF_OTHER, (double)M * (lin_bytes(ctx->emb) / ctx->emb.n + 4.0 * c.hidden), 0,
                     [&] { return launch_embed(ctx->stream, ctx->emb, tokens_dev + r0, M, h, ctx->at<uint32_t>(ctx->L.flags)); }));
    } else {
      LFM3_TRY(launch_bf16_to_f32(ctx->stream, hidden_dev + (size_t)r0 * H, M, H, h));
    }
    st = run_layers(ctx, rows, r0, hidden_out_dev ? hidden_out_dev + (size_t)r0 * H : nullptr);
    if (st != LFM3_OK) return st;
    ctx->len[slot] += M;
    if (r0 + M == n_rows) {
      st = head(ctx, ctx->at<f16_t>(ctx->L.xf) + (size_t)(M - 1) * H, 1, logits_last_dev, argmax_last_dev);
      if (st != LFM3_OK) return st;
    }
  }
  LFM3_TRY(prof_close(ctx));
  return LFM3_OK;
}

lfm3_status lfm3_decode_batch(lfm3_ctx* ctx, int32_t n, const int32_t* slots_host, const int32_t* tokens_dev,
                              const uint16_t* hidden_dev, float* logits_dev, int32_t* argmax_dev, float* hidden_out_dev) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  const lfm3_config& c = ctx->cfg;
  if (n < 1 || n > std::min(c.max_slots, (int)kMaxBatch)) return ctx->fail(LFM3_ERR_ARG, "batch n outside [1, min(max_slots, 64)]");
  if (!slots_host) return ctx->fail(LFM3_ERR_ARG, "slots_host is NULL");
  if ((tokens_dev == nullptr) == (hidden_dev == nullptr)) return ctx->fail(LFM3_ERR_ARG, "pass exactly one of tokens and hidden");
  if (tokens_dev && !c.has_embedding) return ctx->fail(LFM3_ERR_ARG, "token input needs has_embedding = 1");
  if ((logits_dev || argmax_dev) && !c.has_embedding) return ctx->fail(LFM3_ERR_ARG, "logits need the tied head (has_embedding = 1)");
  if (ctx->capture && n > ctx->capture_rows) return ctx->fail(LFM3_ERR_CAPACITY, "capture buffer holds fewer rows than this call");
  std::vector<char> seen(c.max_slots, 0);
  int budget = (int)ctx->free_pages.size();
  std::vector<std::pair<int, int>> writes;
  for (int b = 0; b < n; ++b) {
    const int sl = slots_host[b];
    if (sl < 0 || sl >= c.max_slots) return ctx->fail(LFM3_ERR_SLOT, "slot " + std::to_string(sl) + " outside [0, max_slots)");
    if (seen[sl]) return ctx->fail(LFM3_ERR_ARG, "slot " + std::to_string(sl) + " appears twice in one step");
    if (ctx->pending[sl]) return ctx->fail(LFM3_ERR_ARG, "slot " + std::to_string(sl) + " has an uncommitted verify window");
    seen[sl] = 1;
    if (ctx->len[sl] + 1 > c.max_ctx) return ctx->fail(LFM3_ERR_CAPACITY, "slot " + std::to_string(sl) + " is at max_ctx");
    if (!reserve_pages(ctx, sl, ctx->len[sl] + 1, writes, budget)) return ctx->fail(LFM3_ERR_CAPACITY, "KV page pool exhausted");
  }
  Rows rows{};
  rows.n = n; rows.mode = 1;
  for (int b = 0; b < n; ++b) {
    rows.slot[b] = slots_host[b];
    rows.pos[b] = ctx->len[slots_host[b]];
    lfm3_status st = commit_pages(ctx, slots_host[b], ctx->len[slots_host[b]] + 1);
    if (st != LFM3_OK) return st;
  }
  float* h = ctx->at<float>(ctx->L.h);
  if (tokens_dev) {
    LFM3_TRY(timed(ctx, LFM3_PROF_OTHER, (double)n * (lin_bytes(ctx->emb) / ctx->emb.n + 4.0 * c.hidden), 0,
                   [&] { return launch_embed(ctx->stream, ctx->emb, tokens_dev, n, h, ctx->at<uint32_t>(ctx->L.flags)); }));
  } else {
    LFM3_TRY(launch_bf16_to_f32(ctx->stream, hidden_dev, n, c.hidden, h));
  }
  lfm3_status st = run_decode(ctx, rows, hidden_out_dev, logits_dev, argmax_dev);
  if (st != LFM3_OK) return st;
  for (int b = 0; b < n; ++b) ctx->len[slots_host[b]] += 1;
  LFM3_TRY(prof_close(ctx));
  return LFM3_OK;
}

lfm3_status lfm3_state_bytes(const lfm3_ctx* ctx, int32_t length, size_t* bytes) {
  if (!ctx || !bytes) { g_err = "NULL argument"; return LFM3_ERR_ARG; }
  if (length < 0 || length > ctx->cfg.max_ctx) { g_err = "length outside [0, max_ctx]"; return LFM3_ERR_ARG; }
  *bytes = state_layout(ctx->cfg, ctx->L, length).total;
  return LFM3_OK;
}

lfm3_status lfm3_save_state(lfm3_ctx* ctx, int32_t slot, void* dst_dev, size_t dst_bytes, int32_t* length_out) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  if (slot < 0 || slot >= ctx->cfg.max_slots) return ctx->fail(LFM3_ERR_SLOT, "slot " + std::to_string(slot) + " outside [0, max_slots)");
  if (!dst_dev || (uintptr_t)dst_dev % 256) return ctx->fail(LFM3_ERR_ARG, "dst_dev must be a 256-byte-aligned device pointer");
  if (ctx->pending[slot]) return ctx->fail(LFM3_ERR_ARG, "slot " + std::to_string(slot) + " has an uncommitted verify window");
  const int length = ctx->len[slot];
  const size_t need = state_layout(ctx->cfg, ctx->L, length).total;
  if (dst_bytes < need) return ctx->fail(LFM3_ERR_CAPACITY, "state buffer " + std::to_string(dst_bytes) + " B < " + std::to_string(need) + " B");
  lfm3_status st = move_state(ctx, slot, length, (uint8_t*)dst_dev, 0);
  if (st != LFM3_OK) return st;
  if (length_out) *length_out = length;
  return LFM3_OK;
}

lfm3_status lfm3_load_state(lfm3_ctx* ctx, int32_t slot, const void* src_dev, size_t src_bytes, int32_t length) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  const lfm3_config& c = ctx->cfg;
  if (slot < 0 || slot >= c.max_slots) return ctx->fail(LFM3_ERR_SLOT, "slot " + std::to_string(slot) + " outside [0, max_slots)");
  if (!src_dev || (uintptr_t)src_dev % 256) return ctx->fail(LFM3_ERR_ARG, "src_dev must be a 256-byte-aligned device pointer");
  if (length < 0 || length > c.max_ctx) return ctx->fail(LFM3_ERR_CAPACITY, "length outside [0, max_ctx]");
  const size_t need = state_layout(c, ctx->L, length).total;
  if (src_bytes < need) return ctx->fail(LFM3_ERR_ARG, "state buffer " + std::to_string(src_bytes) + " B < " + std::to_string(need) + " B");
  if (n_of_type(c, LFM3_LAYER_FULL) > 0) {
    const int need_pages = (length + kPageTokens - 1) / kPageTokens;
    if (need_pages > (int)ctx->free_pages.size() + (int)ctx->pages[slot].size())
      return ctx->fail(LFM3_ERR_CAPACITY, "KV page pool exhausted");
  }
  // empty the slot, lease pages for `length` positions, then copy the state in
  for (auto it = ctx->pages[slot].rbegin(); it != ctx->pages[slot].rend(); ++it) ctx->free_pages.push_back(*it);
  ctx->pages[slot].clear();
  ctx->len[slot] = 0;
  ctx->pending[slot] = 0;
  lfm3_status st = commit_pages(ctx, slot, length);
  if (st != LFM3_OK) return st;
  st = move_state(ctx, slot, length, (uint8_t*)const_cast<void*>(src_dev), 1);
  if (st != LFM3_OK) return st;
  ctx->len[slot] = length;
  return LFM3_OK;
}

lfm3_status lfm3_verify(lfm3_ctx* ctx, int32_t slot, const int32_t* tokens_dev, int32_t n_rows, float* logits_dev,
                        int32_t* argmax_dev) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  const lfm3_config& c = ctx->cfg;
  if (slot < 0 || slot >= c.max_slots) return ctx->fail(LFM3_ERR_SLOT, "slot " + std::to_string(slot) + " outside [0, max_slots)");
  if (!c.has_embedding) return ctx->fail(LFM3_ERR_ARG, "verify windows need the embedding and tied head");
  if (!tokens_dev || (!logits_dev && !argmax_dev)) return ctx->fail(LFM3_ERR_ARG, "tokens and an output are required");
  if (n_rows < 1 || n_rows > std::min(kMaxVerify, c.max_chunk))
    return ctx->fail(LFM3_ERR_ARG, "verify rows outside [1, min(16, max_chunk)]");
  if (ctx->pending[slot]) return ctx->fail(LFM3_ERR_ARG, "slot " + std::to_string(slot) + " has an uncommitted verify window");
  if (ctx->capture) return ctx->fail(LFM3_ERR_ARG, "layer capture is not available in a verify pass");
  if ((int64_t)ctx->len[slot] + n_rows > c.max_ctx) return ctx->fail(LFM3_ERR_CAPACITY, "window runs past max_ctx");
  std::vector<std::pair<int, int>> writes;
  int budget = (int)ctx->free_pages.size();
  if (!reserve_pages(ctx, slot, ctx->len[slot] + n_rows, writes, budget)) return ctx->fail(LFM3_ERR_CAPACITY, "KV page pool exhausted");
  lfm3_status st = commit_pages(ctx, slot, ctx->len[slot] + n_rows);
  if (st != LFM3_OK) return st;
  const Layout& L = ctx->L;
  const int n_conv = n_of_type(c, LFM3_LAYER_CONV);
  if (L.conv_slot)
    LFM3_TRY(launch_copy(ctx->stream, ctx->at<f16_t>(L.vpre) + (size_t)slot * L.conv_slot,
                         ctx->at<f16_t>(L.conv_state) + (size_t)slot * L.conv_slot, L.conv_slot * 2));
  LFM3_TRY(timed(ctx, LFM3_PROF_OTHER, (double)n_rows * (lin_bytes(ctx->emb) / ctx->emb.n + 4.0 * c.hidden), 0, [&] {
    return launch_embed(ctx->stream, ctx->emb, tokens_dev, n_rows, ctx->at<float>(L.h), ctx->at<uint32_t>(L.flags));
  }));
  Rows rows{};
  rows.n = n_rows; rows.mode = 0; rows.slot0 = slot; rows.pos0 = ctx->len[slot];
  ctx->verify_z = ctx->at<f16_t>(L.vz) + (size_t)slot * n_conv * kMaxVerify * c.hidden;
  st = run_layers(ctx, rows, 0, nullptr);
  ctx->verify_z = nullptr;
  if (st != LFM3_OK) return st;
  st = head(ctx, ctx->at<f16_t>(L.xf), n_rows, logits_dev, argmax_dev);
  if (st != LFM3_OK) return st;
  ctx->len[slot] += n_rows;
  ctx->pending[slot] = n_rows;
  LFM3_TRY(prof_close(ctx));
  return LFM3_OK;
}

lfm3_status lfm3_commit(lfm3_ctx* ctx, int32_t slot, int32_t n_accept) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  const lfm3_config& c = ctx->cfg;
  if (slot < 0 || slot >= c.max_slots) return ctx->fail(LFM3_ERR_SLOT, "slot " + std::to_string(slot) + " outside [0, max_slots)");
  const int n = ctx->pending[slot];
  if (n == 0) return ctx->fail(LFM3_ERR_ARG, "slot " + std::to_string(slot) + " has no verify window to commit");
  if (n_accept < 0 || n_accept > n) return ctx->fail(LFM3_ERR_ARG, "n_accept outside [0, window rows]");
  const Layout& L = ctx->L;
  const int n_conv = n_of_type(c, LFM3_LAYER_CONV);
  if (n_accept < n)
    LFM3_TRY(launch_conv_commit(ctx->stream, ctx->at<f16_t>(L.conv_state) + (size_t)slot * L.conv_slot,
                                ctx->at<f16_t>(L.vpre) + (size_t)slot * L.conv_slot,
                                ctx->at<f16_t>(L.vz) + (size_t)slot * n_conv * kMaxVerify * c.hidden, kMaxVerify,
                                n_accept, n_conv, c.hidden, c.conv_taps));
  const int len = ctx->len[slot] - n + n_accept;
  ctx->len[slot] = len;
  ctx->pending[slot] = 0;
  // pages past the accepted rows go back to the pool (their stale rows are never read: a later
  // position's key and value are written before any query sees them)
  auto& pg = ctx->pages[slot];
  const int keep = n_of_type(c, LFM3_LAYER_FULL) ? (len + kPageTokens - 1) / kPageTokens : 0;
  while ((int)pg.size() > keep) {
    ctx->free_pages.push_back(pg.back());
    pg.pop_back();
  }
  return LFM3_OK;
}

lfm3_status lfm3_reset_slot(lfm3_ctx* ctx, int32_t slot) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  if (slot < 0 || slot >= ctx->cfg.max_slots) return ctx->fail(LFM3_ERR_SLOT, "slot " + std::to_string(slot) + " outside [0, max_slots)");
  const Layout& L = ctx->L;
  if (L.conv_slot) LFM3_TRY(launch_zero(ctx->stream, ctx->at<f16_t>(L.conv_state) + (size_t)slot * L.conv_slot, L.conv_slot * 2));
  for (auto it = ctx->pages[slot].rbegin(); it != ctx->pages[slot].rend(); ++it) ctx->free_pages.push_back(*it);
  ctx->pages[slot].clear();
  ctx->len[slot] = 0;
  ctx->pending[slot] = 0;
  return LFM3_OK;
}

int32_t lfm3_slot_length(const lfm3_ctx* ctx, int32_t slot) {
  if (!ctx || slot < 0 || slot >= ctx->cfg.max_slots) return -1;
  return ctx->len[slot];
}

lfm3_status lfm3_synchronize(lfm3_ctx* ctx) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  LFM3_TRY(hipStreamSynchronize(ctx->stream));
  uint32_t flags = 0;
  LFM3_TRY(hipMemcpy(&flags, ctx->at<uint32_t>(ctx->L.flags), 4, hipMemcpyDeviceToHost));
  if (flags == 0) return LFM3_OK;
  LFM3_TRY(launch_zero(ctx->stream, ctx->at<void>(ctx->L.flags), 256));
  LFM3_TRY(hipStreamSynchronize(ctx->stream));
  return ctx->fail(LFM3_ERR_ARG, "a token id outside [0, vocab) reached the embedding since the last synchronize "
                                 "(its row was embedded as zeros)");
}

int32_t lfm3_free_pages(const lfm3_ctx* ctx) { return ctx ? (int32_t)ctx->free_pages.size() : -1; }

const char* lfm3_last_error(const lfm3_ctx* ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

lfm3_status lfm3_capture_layers(lfm3_ctx* ctx, float* dev_buf, int32_t max_rows) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  if (dev_buf && max_rows < 1) return ctx->fail(LFM3_ERR_ARG, "max_rows must be >= 1");
  ctx->capture = dev_buf;
  ctx->capture_rows = dev_buf ? max_rows : 0;
  return LFM3_OK;
}

lfm3_status lfm3_dequant_rows(lfm3_ctx* ctx, const char* name, int32_t row0, int32_t n_rows, float* out_f32_dev, uint16_t* out_f16_dev) {
  if (!ctx || !name) { g_err = "NULL argument"; return LFM3_ERR_ARG; }
  auto it = ctx->lin_by_name.find(name);
  if (it == ctx->lin_by_name.end()) return ctx->fail(LFM3_ERR_ARG, std::string("no quantized linear named ") + name);
  const QLinear& w = it->second;
  if (row0 < 0 || n_rows < 1 || row0 + n_rows > w.n) return ctx->fail(LFM3_ERR_ARG, "rows outside the tensor");
  LFM3_TRY(launch_dequant_rows(ctx->stream, w, row0, n_rows, out_f32_dev, (f16_t*)out_f16_dev));
  return LFM3_OK;
}

lfm3_status lfm3_linear(lfm3_ctx* ctx, const char* name, int32_t path, const uint16_t* x_dev, int32_t rows, float* y_dev) {
  if (!ctx || !name || !x_dev || !y_dev) { g_err = "NULL argument"; return LFM3_ERR_ARG; }
  auto it = ctx->lin_by_name.find(name);
  if (it == ctx->lin_by_name.end()) return ctx->fail(LFM3_ERR_ARG, std::string("no quantized linear named ") + name);
  const QLinear& w = it->second;
  if (path == 0) {
    if (rows < 1 || rows > 8) return ctx->fail(LFM3_ERR_ARG, "GEMV rows must be in [1, 8]");
    GemvArgs g{};
    g.w = w; g.x = x_dev; g.ldx = w.k; g.batch = rows; g.epi = GEMV_STORE; g.yf = y_dev; g.ldy = w.n;
    LFM3_TRY(launch_gemv(ctx->stream, g));
  } else if (path == 2) {
    if (rows < 1 || rows > 8) return ctx->fail(LFM3_ERR_ARG, "GEMV rows must be in [1, 8]");
    GemvArgs g{};
    g.w = w; g.x = x_dev; g.ldx = w.k; g.batch = rows; g.epi = GEMV_SWIGLU; g.y = (f16_t*)y_dev; g.ldy = w.n / 2;
    LFM3_TRY(launch_gemv(ctx->stream, g));
  } else if (path == 1 || path == 3 || path == 6) {
    if (rows < 1) return ctx->fail(LFM3_ERR_ARG, "GEMM rows must be >= 1");
    auto gt = ctx->gemm_by_name.find(name);
    if (gt == ctx->gemm_by_name.end()) return ctx->fail(LFM3_ERR_ARG, std::string(name) + " has no GEMM copy (the head is decode-only)");
    GemmArgs g{};
    g.w = gt->second; g.x = x_dev; g.ldx = w.k; g.m = rows;
    if (path == 6) {   // dequantise the codes in the K loop instead of the fp16 copy
      if (!g.w.codes) return ctx->fail(LFM3_ERR_ARG, std::string(name) + " has no re-tiled codes (stored as bf16, NVFP4 or block-FP8)");
      g.w.w16 = nullptr;
    }
    if (path == 3) { g.epi = GEMM_SWIGLU; g.y = (f16_t*)y_dev; g.ldy = w.n / 2; }
    else { g.epi = GEMM_STORE; g.yf = y_dev; g.ldy = w.n; }
    LFM3_TRY(launch_gemm(ctx->stream, g));
  } else if (path == 4 || path == 5) {
    if (rows < 1 || rows > 64) return ctx->fail(LFM3_ERR_ARG, "decode MFMA rows must be in [1, 64]");
    auto gt = ctx->gemm_by_name.find(name);
    if (gt == ctx->gemm_by_name.end()) return ctx->fail(LFM3_ERR_ARG, std::string(name) + " has no GEMM copy (the head is decode-only)");
    GemvArgs g{};
    g.w = w; g.x = x_dev; g.ldx = w.k; g.batch = rows;
    if (path == 5) { g.epi = GEMV_SWIGLU; g.y = (f16_t*)y_dev; g.ldy = w.n / 2; }
    else { g.epi = GEMV_STORE; g.yf = y_dev; g.ldy = w.n; }
    LFM3_TRY(launch_sgemm(ctx->stream, gt->second, g));
  } else {
    return ctx->fail(LFM3_ERR_ARG, "path must be 0..6");
  }
  return LFM3_OK;
}

}  // extern "C"

namespace {

// The attention-core hook. part / part_floats: where the decode split partials go (the context's
// workspace, or the no-allocation entry point's static scratch); pt_host: a host copy of the
// page table to check (NULL: read the device table back).
lfm3_status attention_impl(lfm3_ctx* ctx, const lfm3_attn_io* io, float* part, size_t part_floats,
                           const int32_t* pt_host) {
  if (!ctx || !io) { g_err = "NULL argument"; return LFM3_ERR_ARG; }
  const lfm3_config& c = ctx->cfg;
  const Layout& L = ctx->L;
  const int n = io->n_rows;
  if (!io->slots_host || !io->pos_host || !io->qkvg_dev || !io->q_norm_dev || !io->k_norm_dev || !io->k_cache_dev ||
      !io->v_cache_dev || !io->out_dev)
    return ctx->fail(LFM3_ERR_ARG, "NULL buffer in lfm3_attn_io");
  const int width = (c.n_q_heads + 2 * c.n_kv_heads) * kHeadDim + c.n_q_heads;
  if (io->ld < width) return ctx->fail(LFM3_ERR_ARG, "ld below the qkvg row width");
  if (io->n_slots < 1) return ctx->fail(LFM3_ERR_ARG, "n_slots must be >= 1");
  const bool decode = io->decode != 0, sliding = io->sliding != 0;
  if (decode && (n < 1 || n > std::min(c.max_slots, (int)kMaxBatch)))
    return ctx->fail(LFM3_ERR_ARG, "decode rows outside [1, min(max_slots, 64)]");
  if (!decode && (n < 1 || n > L.max_rows)) return ctx->fail(LFM3_ERR_ARG, "prefill rows outside [1, max(max_chunk, max_slots)]");
  const int nrow_pos = decode ? n : 1;
  std::vector<char> seen(io->n_slots, 0);
  int last_pos_max = 0;
  for (int b = 0; b < nrow_pos; ++b) {
    const int sl = io->slots_host[b], p = io->pos_host[b];
    if (sl < 0 || sl >= io->n_slots) return ctx->fail(LFM3_ERR_ARG, "slot outside [0, n_slots)");
    if (seen[sl]) return ctx->fail(LFM3_ERR_ARG, "slot appears twice in one decode launch");
    seen[sl] = 1;
    const int last = decode ? p : p + n - 1;
    if (p < 0 || (int64_t)last >= c.max_ctx) return ctx->fail(LFM3_ERR_ARG, "position outside [0, max_ctx)");
    last_pos_max = std::max(last_pos_max, last);
  }
  KvRef kv{};
  kv.k = (f16_t*)io->k_cache_dev;
  kv.v = (f16_t*)io->v_cache_dev;
  if (sliding) {
    const int need = decode ? c.window : c.window + n - 1;
    if (io->ring_rows < need) return ctx->fail(LFM3_ERR_ARG, "ring_rows below what the window and pass need");
    kv.ring = io->ring_rows;
  } else {
    if (!io->page_table_dev || io->max_pages < 1 || io->max_pages > 8192 || io->n_pool_pages < 1)
      return ctx->fail(LFM3_ERR_ARG, "full layers need a page table, max_pages in [1, 8192] and n_pool_pages >= 1");
    if (last_pos_max / kPageTokens >= io->max_pages) return ctx->fail(LFM3_ERR_ARG, "positions past the page table row");
    std::vector<int32_t> pt_copy;
    const int32_t* pt = pt_host;
    if (!pt) {
      pt_copy.resize((size_t)io->n_slots * io->max_pages);
      LFM3_TRY(hipStreamSynchronize(ctx->stream));
      LFM3_TRY(hipMemcpy(pt_copy.data(), io->page_table_dev, pt_copy.size() * 4, hipMemcpyDeviceToHost));
      pt = pt_copy.data();
    }
    for (int b = 0; b < nrow_pos; ++b) {
      const int sl = io->slots_host[b], last = decode ? io->pos_host[b] : io->pos_host[b] + n - 1;
      for (int g = 0; g <= last / kPageTokens; ++g) {
        const int32_t pg = pt[(size_t)sl * io->max_pages + g];
        if (pg < 0 || pg >= io->n_pool_pages) return ctx->fail(LFM3_ERR_ARG, "page table entry outside [0, n_pool_pages)");
      }
    }
    kv.page_table = io->page_table_dev;
    kv.max_pages = io->max_pages;
    kv.ring = 0;
  }
  Rows rows{};
  rows.n = n;
  if (decode) {
    rows.mode = 1;
    for (int b = 0; b < n; ++b) { rows.slot[b] = io->slots_host[b]; rows.pos[b] = io->pos_host[b]; }
  } else {
    rows.mode = 0; rows.slot0 = io->slots_host[0]; rows.pos0 = io->pos_host[0];
  }
  const float* cos_t = ctx->at<float>(sliding ? L.cos_s : L.cos_f);
  const float* sin_t = ctx->at<float>(sliding ? L.sin_s : L.sin_f);
  const int gate_col = (c.n_q_heads + 2 * c.n_kv_heads) * kHeadDim;
  if (decode) {
    AttnDecodeArgs aa{};
    aa.qkvg = io->qkvg_dev; aa.ld = io->ld; aa.gate_col = gate_col;
    aa.q_norm = io->q_norm_dev; aa.k_norm = io->k_norm_dev; aa.cos_t = cos_t; aa.sin_t = sin_t;
    aa.kv = kv; aa.rows = rows; aa.window = sliding ? c.window : 0;
    aa.n_q_heads = c.n_q_heads; aa.n_kv_heads = c.n_kv_heads; aa.eps = c.norm_eps;
    aa.out = (f16_t*)io->out_dev; aa.part = part;
    int ms = 1;
    for (int b = 0; b < n; ++b) {
      const int p = rows.pos[b];
      const int lo = sliding ? std::max(0, p - (c.window - 1)) : 0;
      ms = std::max(ms, (p - lo) / attn_decode_split_keys(sliding, p - lo + 1) + 1);
    }
    if ((size_t)n * c.n_q_heads * ms * kPartStride > part_floats)
      return ctx->fail(LFM3_ERR_CAPACITY, "decode split partials exceed their buffer (" + std::to_string(part_floats) + " floats)");
    aa.max_splits = ms;
    LFM3_TRY(launch_attn_decode(ctx->stream, aa));
  } else {
    QkRopeArgs qa{};
    qa.qkvg = io->qkvg_dev; qa.ld = io->ld; qa.q_norm = io->q_norm_dev; qa.k_norm = io->k_norm_dev;
    qa.cos_t = cos_t; qa.sin_t = sin_t; qa.q_out = ctx->at<f16_t>(L.qrot); qa.kv = kv; qa.rows = rows;
    qa.n_q_heads = c.n_q_heads; qa.n_kv_heads = c.n_kv_heads; qa.eps = c.norm_eps;
    LFM3_TRY(launch_qk_rope(ctx->stream, qa));
    AttnArgs aa{};
    aa.q = qa.q_out; aa.gate = io->qkvg_dev + gate_col; aa.ldg = io->ld; aa.kv = kv; aa.rows = rows;
    aa.window = sliding ? c.window : 0; aa.n_q_heads = c.n_q_heads; aa.n_kv_heads = c.n_kv_heads;
    aa.out = (f16_t*)io->out_dev;
    LFM3_TRY(launch_attn_prefill(ctx->stream, aa));
  }
  return LFM3_OK;
}

}  // namespace

// Split partials of lfm3_attention_noalloc: one file-scope device array per GPU, so that entry
// point allocates nothing. Up to kNoAllocRows decode rows of 16 query heads with up to 65 splits
// each (the most attn_decode_split_keys gives): 4.4 MB, held on every GPU the library runs on
// until the process ends. Every call on a GPU shares its copy; calls that overlap on one GPU race.
constexpr int kNoAllocRows = 8;
constexpr size_t kNoAllocFloats = (size_t)kNoAllocRows * 16 * 65 * kPartStride;
static __device__ __align__(256) float scratch[kNoAllocFloats];

namespace {
constexpr int kMaxDevices = 64;
float* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, looked up once per device (host code
// must use this address, never the array's name, which is a host-side stand-in).
lfm3_status noalloc_scratch(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) { g_err = "no usable HIP device"; return LFM3_ERR_DEVICE; }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) { g_err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e); return LFM3_ERR_DEVICE; }
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return LFM3_OK;
}
}  // namespace

extern "C" {

lfm3_status lfm3_attention(lfm3_ctx* ctx, const lfm3_attn_io* io) {
  if (!ctx) { g_err = "NULL argument"; return LFM3_ERR_ARG; }
  const Layout& L = ctx->L;
  return attention_impl(ctx, io, ctx->at<float>(L.part),
                        (size_t)ctx->cfg.max_slots * ctx->cfg.n_q_heads * L.max_splits * kPartStride, nullptr);
}

lfm3_status lfm3_attention_noalloc(lfm3_ctx* ctx, const lfm3_attn_io* io, const int32_t* page_table_host) {
  if (!ctx || !io) { g_err = "NULL argument"; return LFM3_ERR_ARG; }
  if (!io->decode) return ctx->fail(LFM3_ERR_ARG, "lfm3_attention_noalloc runs decode rows only");
  if (io->n_rows < 1 || io->n_rows > kNoAllocRows)
    return ctx->fail(LFM3_ERR_CAPACITY, "lfm3_attention_noalloc takes 1 .. " + std::to_string(kNoAllocRows) + " rows");
  if (!io->sliding && !page_table_host) return ctx->fail(LFM3_ERR_ARG, "full layers need page_table_host");
  float* part = nullptr;
  const lfm3_status st = noalloc_scratch(&part);
  if (st != LFM3_OK) return ctx->fail(st, g_err);
  return attention_impl(ctx, io, part, kNoAllocFloats, io->sliding ? nullptr : page_table_host);
}

lfm3_status lfm3_profile(lfm3_ctx* ctx, int32_t enable) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  if (hipStreamSynchronize(ctx->stream) != hipSuccess) return ctx->fail(LFM3_ERR_DEVICE, "stream sync failed");
  for (auto& r : ctx->prof_recs) { ctx->prof_pool.push_back(r.a); ctx->prof_pool.push_back(r.b); }
  ctx->prof_recs.clear();
  ctx->prof_open = false;
  ctx->prof = enable != 0;
  return LFM3_OK;
}

lfm3_status lfm3_profile_read(lfm3_ctx* ctx, int32_t kind, double* total_ms, int64_t* launches, double* bytes, double* flops) {
  if (!ctx) { g_err = "ctx is NULL"; return LFM3_ERR_ARG; }
  if (kind < 0 || kind >= LFM3_PROF_KINDS) return ctx->fail(LFM3_ERR_ARG, "unknown profile kind");
  if (hipStreamSynchronize(ctx->stream) != hipSuccess) return ctx->fail(LFM3_ERR_DEVICE, "stream sync failed");
  double ms = 0, by = 0, fl = 0;
  int64_t n = 0;
  for (auto& r : ctx->prof_recs) {
    if (r.kind != kind) continue;
    float t = 0;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return ctx->fail(LFM3_ERR_DEVICE, "event timing failed");
    ms += t; by += r.bytes; fl += r.flops; n += r.launches;
  }
  if (total_ms) *total_ms = ms;
  if (launches) *launches = n;
  if (bytes) *bytes = by;
  if (flops) *flops = fl;
  return LFM3_OK;
}

}  // extern "C"
