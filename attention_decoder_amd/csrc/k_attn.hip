// Attention for the LFM3 attention layers on gfx950: flash-style prefill on MFMA and split-K decode.
//
// Both read K/V from the slot's cache: full layers through the page table (16-token pages), sliding
// layers from the per-slot ring. A key j is visible to a query at position p iff j <= p and, on a
// sliding layer, p - j < window ("LFM3-1.7B port", "window_size, with no mask input": absolute query
// position minus key position below 256). Query head h reads KV head h / 4 ("TensorFold PR #1508":
// four query heads a KV head). The output of each head is multiplied by sigmoid(g_h) in fp32 and
// stored fp16 ("LFM3-1.7B port" table row 4 and the fp32-gate paragraph). q, K, V are fp16.
#include "kernels.h"

namespace lfm3 {

LFM3_DEV const f16_t* kv_src(const KvRef& kv, const f16_t* base, int slot, int pos, int kvh, int n_kv) {
  if (kv.ring == 0) {
    const int page = kv.page_table[(size_t)slot * kv.max_pages + pos / kPageTokens];
    return base + (((size_t)page * n_kv + kvh) * kPageTokens + (pos % kPageTokens)) * kHeadDim;
  }
  return base + (((size_t)slot * n_kv + kvh) * kv.ring + (pos % kv.ring)) * kHeadDim;
}

LFM3_DEV float sigmoidf_(float g) { return 1.f / (1.f + __expf(-g)); }

// ---------------------------------------------------------------------------------------------
// prefill: one block per (32 query rows, kv head), 8 waves: wave w is query head 4 * kvh + w % 4 over
// the even (w < 4) or odd (w >= 4) key tiles; the two halves' softmax states are merged at the end.
// Keys are walked in 64-key tiles staged in LDS: the K and V rows of a tile are loaded into
// registers two tiles ahead (keys outside [k_lo, p_last] read a clamped valid key, masked in the
// softmax; no tile past a half's end is loaded) and stored into one of two LDS buffers one tile
// ahead. The page ids of the
// block's key range are staged in LDS once, so no global load result feeds an address in the loop.
// LDS rows are 256 bytes (128 dims) with the 16-byte chunk c of row r stored at chunk c ^ (r & 15),
// which keeps the K reads, the V transpose reads and the stores free of bank conflicts.
// S^T = K Q^T on v_mfma_f32_32x32x16_f16 (keys as rows, queries as columns), so each lane owns one
// query: its softmax statistics need one exchange with lane ^ 32. Key slot r of an S^T sub-tile
// reads key pi(r) (bits 2 and 3 of r swapped) so that a lane's accumulators for P V are 8
// consecutive keys and feed the B operand of O^T += V^T P^T without moving data. The V^T operand
// comes from the row-major V tile through the gfx950 LDS transpose read (ds_read_b64_tr_b16): in
// each 16-lane group, slot j of lane i receives element i % 4 of the 8 bytes addressed by lane
// 4j + i / 4, so lanes addressing 4 consecutive keys x 4 dims deliver 4 keys of one dim per lane.
// ---------------------------------------------------------------------------------------------

constexpr int PKT = 64;                      // keys per staged tile
constexpr int PTILE = PKT * kHeadDim;        // elements of one K or V tile
constexpr int kAttnPrefillLds = 8 * PTILE * 2;   // per key half: two K and two V buffers (bytes)

LFM3_DEV int swz(int r, int c) { return r * kHeadDim + 8 * (c ^ (r & 15)); }   // element offset
// The V tile's swizzle: chunk c of row r at c ^ 4 (r mod 4) ^ 2 ((r / 8) mod 2). A transpose read
// of a wave covers rows R .. R+3 and R+8 .. R+11 (R a multiple of 8) and 4 chunks of them; with this
// swizzle each half-wave's 32 lanes read 32 different 8-byte bank pairs (with the K swizzle rows R
// and R+1 shared their chunks: 4-way conflicts, 6 cycles a read, measured with SQ_LDS_BANK_CONFLICT).
LFM3_DEV int swzv(int r, int c) { return r * kHeadDim + 8 * (c ^ (4 * (r & 3)) ^ (2 * ((r >> 3) & 1))); }

typedef short s16x4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_v lds_s16x4;

template <bool PAGED>
__global__ void __launch_bounds__(512, 1) k_attn_prefill(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) f16_t attn_smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kh = wave >> 2;               // key half: even or odd tiles
  const int tid = threadIdx.x & 255;      // thread within the half
  f16_t* Ks = attn_smem + kh * 4 * PTILE;              // [2][PTILE]
  f16_t* Vs = attn_smem + kh * 4 * PTILE + 2 * PTILE;  // [2][PTILE]
  int* pids = (int*)(attn_smem + 8 * PTILE);
  const int kvh = blockIdx.y;
  const int h = kvh * kQPerKv + (wave & 3);
  const int M = a.rows.n;
  // the causal work grows with the query block: the longest blocks are dispatched first
  const int r0 = (gridDim.x - 1 - blockIdx.x) * 32;
  const int slot = a.rows.slot0;
  const int p_first = a.rows.pos0 + r0;
  const int r_last = min(M - 1, r0 + 31);
  const int p_last = a.rows.pos0 + r_last;
  const int nq = a.n_q_heads, nkv = a.n_kv_heads;

  // this lane's query (column) and its position; rows past M read row M - 1 and are not stored
  const int qr = r0 + (lane & 31);
  const int qpos = a.rows.pos0 + qr;
  const bool qvalid = qr < M;
  f16x8_v qv[8];
  {
    const f16_t* qp = a.q + ((size_t)min(qr, M - 1) * nq + h) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[s] = *(const f16x8_v*)(qp + 16 * s + 8 * (lane >> 5));
  }
  int k_lo = 0;
  if (a.window > 0) k_lo = max(0, p_first - (a.window - 1));
  const int kb0 = k_lo / 32 * 32;
  const int ntiles = (p_last - kb0) / PKT + 1;

  // page ids of the keys [kb0, p_last]
  const int pg0 = kb0 / kPageTokens;
  if constexpr (PAGED) {
    const int32_t* pt = a.kv.page_table + (size_t)slot * a.kv.max_pages;
    for (int i = threadIdx.x; i <= p_last / kPageTokens - pg0; i += 512) pids[i] = pt[pg0 + i];
    __syncthreads();
  }
  auto row_of = [&](int key) -> size_t {
    if constexpr (PAGED) return (((size_t)pids[key / kPageTokens - pg0] * nkv + kvh) * kPageTokens + (key % kPageTokens)) * kHeadDim;
    else return (((size_t)slot * nkv + kvh) * a.kv.ring + (key % a.kv.ring)) * kHeadDim;
  };
  // thread t moves chunks u = t + 256 i (i < 4) of the tile's 64 rows x 16 chunks
  auto gload = [&](int i_loc, u32x4_v (&kr)[4], u32x4_v (&vr)[4]) {
    const int kb = kb0 + (2 * i_loc + kh) * PKT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      const int key = min(max(kb + (u >> 4), k_lo), p_last);
      const size_t o = row_of(key) + 8 * (u & 15);
      kr[i] = *(const u32x4_v*)(a.kv.k + o);
      vr[i] = *(const u32x4_v*)(a.kv.v + o);
    }
  };
  auto sstore = [&](int buf, const u32x4_v (&kr)[4], const u32x4_v (&vr)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      *(u32x4_v*)(Ks + buf * PTILE + swz(u >> 4, u & 15)) = kr[i];
      *(u32x4_v*)(Vs + buf * PTILE + swzv(u >> 4, u & 15)) = vr[i];
    }
  };

  f32x16_v o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[d][v] = 0.f;
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  const float scale = 0.08838834764831845f * 1.4426950408889634f;  // 1/sqrt(128) * log2(e)
  const int ks_r = lane & 31;
  const int kslot = (ks_r & ~12) | ((ks_r & 4) << 1) | ((ks_r & 8) >> 1);
  // transpose-read lane roles: group g = lane / 16, key j = (lane % 16) / 4, dims 4q .. 4q + 3
  const int tg = lane >> 4, tj = (lane & 15) >> 2, tq = lane & 3;

  auto compute = [&](int i_loc) {
    const f16_t* Kt = Ks + (i_loc & 1) * PTILE;
    const f16_t* Vt = Vs + (i_loc & 1) * PTILE;
    const int kb = kb0 + (2 * i_loc + kh) * PKT;
    f32x16_v st[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[sub][v] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const f16x8_v kvv = *(const f16x8_v*)(Kt + swz(32 * sub + kslot, 2 * s + (lane >> 5)));
        st[sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kvv, qv[s], st[sub], 0, 0, 0);
      }
    }
    // acc v of sub-tile sub is key kb + 32 sub + 16(v/8) + 8(lane/32) + v%8
    const bool interior = kb >= k_lo && kb + PKT - 1 <= p_first && (a.window == 0 || p_last - kb < a.window);
    // the running max is kept in scaled units; the tile's max is taken on the raw scores (the
    // scale is positive, so the maximum commutes with it) and the scale enters each exponent
    // through one fma
    float sv[2][16];
    float mloc = -__builtin_huge_valf();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = st[sub][v];
        if (!interior) {
          const int j = kb + 32 * sub + 16 * (v >> 3) + 8 * (lane >> 5) + (v & 7);
          bool vis = j >= k_lo && j <= qpos;
          if (a.window > 0) vis = vis && (qpos - j) < a.window;
          x = vis ? x : -__builtin_huge_valf();
        }
        sv[sub][v] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc * scale);
    const bool none = m_new == -__builtin_huge_valf();
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float lsum = 0.f;
    f16x8_v pv[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pr = none ? 0.f : exp2f(fmaf(sv[sub][v], scale, -m_new));
        lsum += pr;
        pv[sub][v >> 3][v & 7] = (_Float16)pr;
      }
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    // O is rescaled only when some lane's max moved (alpha is exactly 1 otherwise)
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[d][v] *= alpha;
    }
    // O^T[dim][query] += V^T[dim][keys] P^T[keys][query]
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int kr = 32 * sub + 16 * t2 + 8 * (tg >> 1) + tj;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int c = 4 * d + 2 * (tg & 1) + (tq >> 1);
          const int half = 4 * (tq & 1);
          const s16x4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + swzv(kr, c) + half));
          const s16x4_v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + swzv(kr + 4, c) + half));
          const f16x8_v vt = __builtin_bit_cast(f16x8_v, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt, pv[sub][t2], o[d], 0, 0, 0);
        }
      }
  };

  // local tile i + 1 is stored while local tile i is computed; local tile i + 3 is loaded into the
  // registers the store freed (register sets A and B alternate, so nothing is copied across the
  // loop edge). Both halves run the same number of iterations (a past-the-end tile of the odd half
  // is not computed) so that they meet at every barrier; tiles past a half's end are not loaded
  // (a spare load would hold the wave until it returns), and their stores are never read.
  const int nloc = (ntiles + 1) / 2;
  u32x4_v kA[4], vA[4], kB[4] = {}, vB[4] = {};
  auto live = [&](int i_loc) { return 2 * i_loc + kh < ntiles; };
  gload(0, kA, vA);
  sstore(0, kA, vA);
  if (live(1)) gload(1, kA, vA);
  if (live(2)) gload(2, kB, vB);
  __syncthreads();
  for (int i = 0; i < nloc; i += 2) {
    sstore(1, kA, vA);
    if (live(i + 3)) gload(i + 3, kA, vA);
    if (live(i)) compute(i);
    __syncthreads();
    if (i + 1 >= nloc) break;
    sstore(0, kB, vB);
    if (live(i + 4)) gload(i + 4, kB, vB);
    if (live(i + 1)) compute(i + 1);
    __syncthreads();
  }

  // merge the odd half's state into the even half's (the tile buffers are free now)
  float* mb = (float*)attn_smem;   // [4 heads][66][64 lanes]: m, l, o
  float* mine = mb + (size_t)(wave & 3) * 66 * 64 + lane;
  if (kh == 1) {
    mine[0] = m_run;
    mine[64] = l_run;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) mine[64 * (2 + 16 * d + v)] = o[d][v];
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float m1 = mine[0], l1 = mine[64];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -__builtin_huge_valf() ? 0.f : exp2f(m_run - m);
    const float a1 = m1 == -__builtin_huge_valf() ? 0.f : exp2f(m1 - m);
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[d][v] = o[d][v] * a0 + mine[64 * (2 + 16 * d + v)] * a1;
  }

  if (!qvalid) return;
  const float gate = sigmoidf_(a.gate[(size_t)qr * a.ldg + h]);
  const float inv = l_run > 0.f ? gate / l_run : 0.f;
  f16_t* dst = a.out + (size_t)qr * nq * kHeadDim + (size_t)h * kHeadDim;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int dim = 32 * d + 8 * v4 + 4 * (lane >> 5);
      const uint32_t w0 = pack_h2(o[d][4 * v4] * inv, o[d][4 * v4 + 1] * inv);
      const uint32_t w1 = pack_h2(o[d][4 * v4 + 2] * inv, o[d][4 * v4 + 3] * inv);
      *(uint2*)(dst + dim) = make_uint2(w0, w1);
    }
}

hipError_t launch_attn_prefill(hipStream_t s, const AttnArgs& a) {
  if (a.rows.n <= 0) return hipSuccess;
  // per key half two K and two V tiles, then the page ids of up to the whole page table row
  const size_t lds = kAttnPrefillLds + (a.kv.ring == 0 ? (size_t)a.kv.max_pages * sizeof(int) : 0);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static size_t lds_set[2] = {0, 0};
  const bool paged = a.kv.ring == 0;
  const void* fn = paged ? (const void*)k_attn_prefill<true> : (const void*)k_attn_prefill<false>;
  if (lds > lds_set[paged]) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_set[paged] = lds;
  }
  const dim3 grid((a.rows.n + 31) / 32, a.n_kv_heads);
  if (paged) hipLaunchKernelGGL(k_attn_prefill<true>, grid, dim3(512), lds, s, a);
  else hipLaunchKernelGGL(k_attn_prefill<false>, grid, dim3(512), lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// decode: block (split, kv head, row); a split is attn_decode_split_keys(row) consecutive visible
// keys (a multiple of 64), walked in 64-key tiles with an online softmax, the next tile's K/V loads
// (and the page ids of the one after) in flight while a tile is computed. The prologue normalises
// and rotates the block's 4 query heads from the raw qkvg row; the block whose split holds the
// current position also forms its key and value (per-head k RMSNorm + RoPE) and stores them in the
// cache. Scores: 4 lanes per key (32 dims each, summed by DPP); wave w is query head 4 kvh + w for
// the softmax and P V (lane = 2 dims). One split: the block writes the gated output. Several:
// partials (max, sum, o) go to the workspace and k_attn_merge, the next launch, combines them (the
// kernel boundary orders the partials' stores before its loads; an in-kernel last-block merge
// would need an agent-scope release and acquire per block, a write-back and an invalidate of the
// L2, which measured slower than the extra launch). With merge_in_consumer set (sliding layers at
// 1-2 rows, at most kFusedMergeSplits splits) the o_proj GEMV merges them in its prologue instead.
// ---------------------------------------------------------------------------------------------

constexpr int TILE = 64;
constexpr int KVS = kHeadDim + 8;   // LDS row stride of the K and V tiles (elements)
constexpr int kMaxMergeSplits = 512;
template <bool PAGED>
LFM3_DEV size_t kv_off(const KvRef& kv, int slot, int pos, int page, int kvh, int n_kv) {
  if constexpr (PAGED) return (((size_t)page * n_kv + kvh) * kPageTokens + (pos % kPageTokens)) * kHeadDim;
  else return (((size_t)slot * n_kv + kvh) * kv.ring + (pos % kv.ring)) * kHeadDim;
}

// a.x * b.x + a.y * b.y + c over fp16 pairs (the words are taken by value: a bit cast of a vector
// element in place was seen to read element 0 for every index)
LFM3_DEV float dot2_h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_v, a), __builtin_bit_cast(f16x2_v, b), c, false);
}

template <bool PAGED>
__global__ void __launch_bounds__(256) k_attn_decode(AttnDecodeArgs a) {
  __shared__ __attribute__((aligned(16))) f16_t kt[(TILE + 1) * KVS];   // row TILE: spare (unused keys)
  __shared__ __attribute__((aligned(16))) f16_t vt[(TILE + 1) * KVS];
  __shared__ __attribute__((aligned(16))) f16_t qs[kQPerKv][kHeadDim];   // the fp16 queries
  __shared__ float sc[kQPerKv][TILE];
  __shared__ __attribute__((aligned(16))) f16_t knew[kHeadDim], vnew[kHeadDim];
  const int split = blockIdx.x, kvh = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slot = a.rows.slot[r], pos = a.rows.pos[r];
  const int nq = a.n_q_heads, nkv = a.n_kv_heads;
  const int k_lo = a.window > 0 ? max(0, pos - (a.window - 1)) : 0;
  const int SK = attn_decode_split_keys(a.window > 0, pos - k_lo + 1);
  const int ns = (pos - k_lo) / SK + 1;
  if (split >= ns) return;
  const int j0 = k_lo + split * SK;
  const int j_end = min(pos, j0 + SK - 1);          // last key of the split
  const int n_tiles = (j_end - j0) / TILE + 1;
  const bool has_new = split == ns - 1;   // the current position is this split's last key
  const int32_t* pt = PAGED ? a.kv.page_table + (size_t)slot * a.kv.max_pages : nullptr;

  // tile loads: thread t moves 16-byte chunks t + 256 q (q < 4) of the 64 key x 16 chunk tile;
  // keys past the split in its last tile read the split's last key (not used)
  auto key_of = [&](int tile, int q) { return min(j0 + tile * TILE + ((tid + 256 * q) >> 4), j_end); };
  int pg[4], pgn[4] = {0, 0, 0, 0};
  u32x4_v kr[4], vr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) pg[q] = PAGED ? pt[key_of(0, q) / kPageTokens] : 0;
  // the step's own query row (issued with the page ids: independent loads)
  const float* row = a.qkvg + (size_t)r * a.ld;
  const int hq = kvh * kQPerKv + wave;
  const float c = a.cos_t[(size_t)pos * kHalfDim + lane];
  const float sn = a.sin_t[(size_t)pos * kHalfDim + lane];
  const float x0 = row[(size_t)hq * kHeadDim + lane], x1 = row[(size_t)hq * kHeadDim + lane + kHalfDim];
  const float qn0 = bf2f(a.q_norm[lane]), qn1 = bf2f(a.q_norm[lane + kHalfDim]);
  // new key (wave 0) / value (wave 1) inputs
  const float* nrow = row + (size_t)(wave == 0 ? nq + kvh : nq + nkv + kvh) * kHeadDim;
  const float y0 = nrow[lane], y1 = nrow[lane + kHalfDim];
  const float kn0 = bf2f(a.k_norm[lane]), kn1 = bf2f(a.k_norm[lane + kHalfDim]);
  const float graw = row[a.gate_col + hq];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const size_t o = kv_off<PAGED>(a.kv, slot, key_of(0, q), pg[q], kvh, nkv) + 8 * ((tid + 256 * q) & 15);
    kr[q] = *(const u32x4_v*)(a.kv.k + o);
    vr[q] = *(const u32x4_v*)(a.kv.v + o);
  }
  if (PAGED && n_tiles > 1)
#pragma unroll
    for (int q = 0; q < 4; ++q) pgn[q] = pt[key_of(1, q) / kPageTokens];

  // q heads 4 kvh + w (wave w): per-head RMSNorm + RoPE ("LFM3-1.7B port": partial RoPE on the
  // full layers); lane holds dims lane, lane + 64; q rounded to fp16 as the prefill path stores it
  {
    const float rr = rsqrtf(wave_sum(x0 * x0 + x1 * x1) / (float)kHeadDim + a.eps);
    const float n0 = x0 * rr * qn0, n1 = x1 * rr * qn1;
    qs[wave][lane] = f2h(n0 * c - n1 * sn);
    qs[wave][lane + kHalfDim] = f2h(n1 * c + n0 * sn);
  }
  if (has_new && wave < 2) {
    float o0, o1;
    if (wave == 0) {
      const float rr = rsqrtf(wave_sum(y0 * y0 + y1 * y1) / (float)kHeadDim + a.eps);
      const float n0 = y0 * rr * kn0, n1 = y1 * rr * kn1;
      o0 = n0 * c - n1 * sn;
      o1 = n1 * c + n0 * sn;
    } else {
      o0 = y0;
      o1 = y1;
    }
    const int page = PAGED ? pt[pos / kPageTokens] : 0;
    f16_t* dst = (wave == 0 ? a.kv.k : a.kv.v) + kv_off<PAGED>(a.kv, slot, pos, page, kvh, nkv);
    const f16_t h0 = f2h(o0), h1 = f2h(o1);
    dst[lane] = h0;
    dst[lane + kHalfDim] = h1;
    f16_t* t = wave == 0 ? knew : vnew;
    t[lane] = h0;
    t[lane + kHalfDim] = h1;
  }

  const float scale = 0.08838834764831845f;
  float m_run = -__builtin_huge_valf(), l_run = 0.f, o0 = 0.f, o1 = 0.f;
  const int d0 = 2 * lane;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int tj = j0 + tile * TILE;
    const int nk = min(TILE, j_end - tj + 1);
    // 1. the tile into LDS: keys past the split and the current position go to the spare row,
    //    the current position's row comes from knew / vnew
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, key = idx >> 4, c8 = idx & 15;
      const int row_l = (key < nk && tj + key != pos) ? key : TILE;
      *(u32x4_v*)(kt + row_l * KVS + 8 * c8) = kr[q];
      *(u32x4_v*)(vt + row_l * KVS + 8 * c8) = vr[q];
    }
    if (has_new && pos >= tj && pos < tj + TILE && tid < 32) {
      const int kk = pos - tj;
      if (tid < 16) *(u32x4_v*)(kt + kk * KVS + 8 * tid) = *(const u32x4_v*)(knew + 8 * tid);
      else *(u32x4_v*)(vt + kk * KVS + 8 * (tid - 16)) = *(const u32x4_v*)(vnew + 8 * (tid - 16));
    }
    __syncthreads();
    // 2. the next tile's loads and the page ids one further, only where the split has that tile
    //    (a spare load would hold the block until it returns)
    if (tile + 1 < n_tiles) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t o = kv_off<PAGED>(a.kv, slot, key_of(tile + 1, q), pgn[q], kvh, nkv) + 8 * ((tid + 256 * q) & 15);
        kr[q] = *(const u32x4_v*)(a.kv.k + o);
        vr[q] = *(const u32x4_v*)(a.kv.v + o);
      }
    }
    if (PAGED && tile + 2 < n_tiles)
#pragma unroll
      for (int q = 0; q < 4; ++q) pgn[q] = pt[key_of(tile + 2, q) / kPageTokens];
    // 3. scores: thread -> key t / 4, dims [32 (t % 4), + 32) for the 4 heads, as fp16 pair dot
    //    products with fp32 accumulation; sum over 4 lanes
    {
      const int key = tid >> 2, qd = tid & 3;
      float d[kQPerKv] = {0.f, 0.f, 0.f, 0.f};
      const f16_t* kp = kt + key * KVS + 32 * qd;
#pragma unroll
      for (int e8 = 0; e8 < 4; ++e8) {
        const u32x4_v v = *(const u32x4_v*)(kp + 8 * e8);
#pragma unroll
        for (int hh = 0; hh < kQPerKv; ++hh) {
          const u32x4_v qv = *(const u32x4_v*)(&qs[hh][32 * qd + 8 * e8]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            d[hh] = dot2_h(v[e], qv[e], d[hh]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < kQPerKv; ++hh) {
        d[hh] += dpp_mov<0xb1>(d[hh]);
        d[hh] += dpp_mov<0x4e>(d[hh]);
      }
      if (qd == 0)
#pragma unroll
        for (int hh = 0; hh < kQPerKv; ++hh) sc[hh][key] = key < nk ? d[hh] * scale : -__builtin_huge_valf();
    }
    __syncthreads();
    // 4. online softmax for head `wave` over the tile (lane = key), then P V with lane = 2 dims
    const float v_ = sc[wave][lane];
    const float m_new = fmaxf(m_run, warp_max(v_));        // finite: every tile has a visible key
    const float alpha = __expf(m_run - m_new);
    const float p = v_ == -__builtin_huge_valf() ? 0.f : __expf(v_ - m_new);
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
    sc[wave][lane] = p;   // each wave rewrites only its own head's row, read back by itself
    o0 *= alpha;
    o1 *= alpha;
    for (int kk = 0; kk < nk; ++kk) {
      const float pk = sc[wave][kk];
      const uint32_t vv = *(const uint32_t*)(vt + kk * KVS + d0);
      o0 = fmaf(pk, h2f((f16_t)(vv & 0xffffu)), o0);
      o1 = fmaf(pk, h2f((f16_t)(vv >> 16)), o1);
    }
  }
  const int h = hq;
  const float gate = sigmoidf_(graw);
  f16_t* out = a.out + (size_t)r * nq * kHeadDim + (size_t)h * kHeadDim;
  if (ns == 1) {
    const float inv = gate / l_run;
    *(uint32_t*)(out + d0) = pack_h2(o0 * inv, o1 * inv);
    return;
  }
  // 5. partials [o (128) | max | sum | pad], merged by k_attn_merge
  float* part = a.part + (((size_t)r * nq + h) * a.max_splits + split) * kPartStride;
  if (lane == 0) { part[kHeadDim] = m_run; part[kHeadDim + 1] = l_run; }
  *(float2*)(part + d0) = make_float2(o0, o1);
}

// Merge of a row's split partials: block (kv head, row), wave w = query head 4 kvh + w, in batches
// of 32 splits with every load of a batch issued at once: lanes 0-31 hold the statistics of split
// s0 + lane; for o, lanes 0-31 take the even splits of the batch and lanes 32-63 the odd ones,
// 4 dims each (lane % 32). Rows with one split were written by k_attn_decode.
__global__ void __launch_bounds__(256) k_attn_merge(AttnDecodeArgs a) {
  __shared__ float wb[kQPerKv][32];
  const int kvh = blockIdx.x, r = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pos = a.rows.pos[r];
  const int nq = a.n_q_heads;
  const int k_lo = a.window > 0 ? max(0, pos - (a.window - 1)) : 0;
  const int ns = (pos - k_lo) / attn_decode_split_keys(a.window > 0, pos - k_lo + 1) + 1;
  if (ns == 1) return;
  const int h = kvh * kQPerKv + wave;
  const float gate = sigmoidf_(a.qkvg[(size_t)r * a.ld + a.gate_col + h]);
  f16_t* out = a.out + (size_t)r * nq * kHeadDim + (size_t)h * kHeadDim;
  float* wbuf = wb[wave];
  const float* ph = a.part + ((size_t)r * nq + h) * a.max_splits * kPartStride;
  const int half = lane >> 5, dq = 4 * (lane & 31);
  float gmx = -__builtin_huge_valf(), lt = 0.f;
  float a4[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int CH = 16;   // splits per lane half per batch
  for (int s0 = 0; s0 < ns; s0 += 2 * CH) {
    const int sS = s0 + (lane & 31);
    const float pm = ph[(size_t)min(sS, ns - 1) * kPartStride + kHeadDim];
    const float pl = ph[(size_t)min(sS, ns - 1) * kPartStride + kHeadDim + 1];
    float4 ov[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) ov[u] = *(const float4*)(ph + (size_t)min(s0 + 2 * u + half, ns - 1) * kPartStride + dq);
    const bool real = sS < ns;
    const float bm = warp_max(real ? pm : -__builtin_huge_valf());
    const float gnew = fmaxf(gmx, bm);
    const float resc = __expf(gmx - gnew);
    const float w = (real && lane < 32) ? __expf(pm - gnew) : 0.f;
    if (lane < 32) wbuf[lane] = w;
    lt = lt * resc + wave_sum(w * pl);
    gmx = gnew;
    // wbuf is written and read by this wave only; LDS operations of a wave stay in order
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int e = 0; e < 4; ++e) a4[e] *= resc;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float wu = wbuf[2 * u + half];   // 0 for splits past ns
      a4[0] = fmaf(wu, ov[u].x, a4[0]);
      a4[1] = fmaf(wu, ov[u].y, a4[1]);
      a4[2] = fmaf(wu, ov[u].z, a4[2]);
      a4[3] = fmaf(wu, ov[u].w, a4[3]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  // the two lane halves hold the even / odd splits of the same 4 dims
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a4[e]), __float_as_uint(a4[e]), false, false);
    a4[e] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (lane < 32) {
    const float inv = lt > 0.f ? gate / lt : 0.f;
    *(uint2*)(out + dq) = make_uint2(pack_h2(a4[0] * inv, a4[1] * inv), pack_h2(a4[2] * inv, a4[3] * inv));
  }
}

hipError_t launch_attn_decode(hipStream_t s, const AttnDecodeArgs& a) {
  if (a.rows.n <= 0) return hipSuccess;
  if (a.max_splits > kMaxMergeSplits) return hipErrorInvalidValue;
  if (a.kv.ring == 0)
    hipLaunchKernelGGL(k_attn_decode<true>, dim3(a.max_splits, a.n_kv_heads, a.rows.n), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_decode<false>, dim3(a.max_splits, a.n_kv_heads, a.rows.n), dim3(256), 0, s, a);
  if (a.max_splits > 1 && !a.merge_in_consumer) hipLaunchKernelGGL(k_attn_merge, dim3(a.n_kv_heads, a.rows.n), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lfm3
