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
// prefill: one block per (32 query rows, kv head); wave w is query head 4 * kvh + w.
// S^T = K Q^T on v_mfma_f32_32x32x16_f16 (keys as rows, queries as columns), so each lane owns one
// query: its softmax statistics need one exchange with lane ^ 32. Key slot r of the S^T tile reads
// key pi(r) (bits 2 and 3 of r swapped) so that a lane's accumulators for P V are 8 consecutive keys
// and feed the B operand of O^T += V^T P^T without moving data.
// ---------------------------------------------------------------------------------------------

constexpr int KT = 32;             // keys per block
constexpr int KS = kHeadDim + 8;   // K tile row stride (elements)
constexpr int VS = KT + 8;         // V^T tile row stride (elements)

__global__ void __launch_bounds__(256) k_attn_prefill(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) f16_t Ks[KT * KS];
  __shared__ __attribute__((aligned(16))) f16_t Vt[kHeadDim * VS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kvh = blockIdx.y;
  const int h = kvh * kQPerKv + wave;
  const int M = a.rows.n;
  const int r0 = blockIdx.x * 32;
  const int slot = a.rows.slot0;
  const int p_first = a.rows.pos0 + r0;
  const int r_last = min(M - 1, r0 + 31);
  const int p_last = a.rows.pos0 + r_last;
  const int nq = a.n_q_heads, nkv = a.n_kv_heads;

  // this lane's query (column) and its position
  const int qr = r0 + (lane & 31);
  const int qpos = a.rows.pos0 + qr;
  const bool qvalid = qr < M;
  f16x8_v qv[8];
  {
    const f16_t* qp = a.q + ((size_t)(qvalid ? qr : 0) * nq + h) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (qvalid) qv[s] = *(const f16x8_v*)(qp + 16 * s + 8 * (lane >> 5));
      else for (int e = 0; e < 8; ++e) qv[s][e] = (_Float16)0.f;
    }
  }
  int k_lo = 0;
  if (a.window > 0) k_lo = max(0, p_first - (a.window - 1));
  const int kb0 = k_lo / KT * KT;

  f32x16_v o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[d][v] = 0.f;
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  const float scale = 0.08838834764831845f * 1.4426950408889634f;  // 1/sqrt(128) * log2(e)
  const int ks_r = lane & 31;
  const int kslot = (ks_r & ~12) | ((ks_r & 4) << 1) | ((ks_r & 8) >> 1);

  for (int kb = kb0; kb <= p_last; kb += KT) {
    // cooperative load: 32 keys x 128 dims for K (row-major) and V (transposed into Vt)
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;   // 512 chunks of 8 dims
      const int key = idx >> 4, c8 = idx & 15;
      const int j = kb + key;
      uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
      if (j >= k_lo && j <= p_last) {
        kv4 = *(const uint4*)(kv_src(a.kv, a.kv.k, slot, j, kvh, nkv) + 8 * c8);
        vv4 = *(const uint4*)(kv_src(a.kv, a.kv.v, slot, j, kvh, nkv) + 8 * c8);
      }
      *(uint4*)(Ks + key * KS + 8 * c8) = kv4;
      const f16_t* ve = (const f16_t*)&vv4;
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(8 * c8 + e) * VS + key] = ve[e];
    }
    __syncthreads();

    // S^T tile: rows = key slots, cols = queries
    f32x16_v st;
#pragma unroll
    for (int v = 0; v < 16; ++v) st[v] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const f16x8_v kvv = *(const f16x8_v*)(Ks + kslot * KS + 16 * s + 8 * (lane >> 5));
      st = __builtin_amdgcn_mfma_f32_32x32x16_f16(kvv, qv[s], st, 0, 0, 0);
    }
    // acc v of this lane is key kb + 16(v/8) + 8(lane/32) + v%8 (after the slot permutation)
    float sv[16];
    float mloc = -__builtin_huge_valf();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = kb + 16 * (v >> 3) + 8 * (lane >> 5) + (v & 7);
      bool vis = j >= k_lo && j <= qpos;
      if (a.window > 0) vis = vis && (qpos - j) < a.window;
      sv[v] = vis ? st[v] * scale : -__builtin_huge_valf();
      mloc = fmaxf(mloc, sv[v]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = m_new == -__builtin_huge_valf() ? 1.f : exp2f(m_run - m_new);
    float lsum = 0.f;
    f16x8_v pv[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = m_new == -__builtin_huge_valf() ? 0.f : exp2f(sv[v] - m_new);
      lsum += p;
      pv[v >> 3][v & 7] = (_Float16)p;
    }
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[d][v] *= alpha;
    // O^T[dim][query] += V^T[dim][keys] P^T[keys][query]
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const f16x8_v vt = *(const f16x8_v*)(Vt + (32 * d + (lane & 31)) * VS + 16 * t + 8 * (lane >> 5));
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt, pv[t], o[d], 0, 0, 0);
      }
    }
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
  hipLaunchKernelGGL(k_attn_prefill, dim3((a.rows.n + 31) / 32, a.n_kv_heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// decode: block (split, kv head, row); 256 keys per split, 4 query heads of one KV head; partials
// (max, sum, o[128]) per (row, head, split) are merged by k_attn_merge.
// ---------------------------------------------------------------------------------------------

constexpr int SPLIT = 256;
int attn_decode_split_keys() { return SPLIT; }

__global__ void __launch_bounds__(256) k_attn_decode(AttnArgs a) {
  __shared__ float qs[kQPerKv][kHeadDim];
  __shared__ float ps[kQPerKv][SPLIT];
  __shared__ float stat[kQPerKv][2];
  const int split = blockIdx.x, kvh = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slot = a.rows.slot[r], pos = a.rows.pos[r];
  const int nq = a.n_q_heads, nkv = a.n_kv_heads;
  const int k_lo = a.window > 0 ? max(0, pos - (a.window - 1)) : 0;
  const int j0 = k_lo + split * SPLIT;
  float* part = a.part + (((size_t)r * nq + kvh * kQPerKv) * a.max_splits + split) * (kHeadDim + 2);
  const size_t head_stride = (size_t)a.max_splits * (kHeadDim + 2);
  if (j0 > pos) {
    if (tid < kQPerKv) { part[tid * head_stride] = -__builtin_huge_valf(); part[tid * head_stride + 1] = 0.f; }
    return;
  }
  const int j1 = min(pos, j0 + SPLIT - 1);
  for (int i = tid; i < kQPerKv * kHeadDim; i += 256) {
    const int hh = i / kHeadDim, d = i % kHeadDim;
    qs[hh][d] = h2f(a.q[((size_t)r * nq + kvh * kQPerKv + hh) * kHeadDim + d]);
  }
  __syncthreads();
  const int j = j0 + tid;
  float sc[kQPerKv] = {0.f, 0.f, 0.f, 0.f};
  if (j <= j1) {
    const uint4* kr = (const uint4*)kv_src(a.kv, a.kv.k, slot, j, kvh, nkv);
#pragma unroll 4
    for (int c = 0; c < kHeadDim / 8; ++c) {
      const uint4 v = kr[c];
      const f16_t* e = (const f16_t*)&v;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float kf = h2f(e[t]);
#pragma unroll
        for (int hh = 0; hh < kQPerKv; ++hh) sc[hh] = fmaf(qs[hh][8 * c + t], kf, sc[hh]);
      }
    }
  }
  const float scale = 0.08838834764831845f;
#pragma unroll
  for (int hh = 0; hh < kQPerKv; ++hh) ps[hh][tid] = j <= j1 ? sc[hh] * scale : -__builtin_huge_valf();
  __syncthreads();
  {
    // wave w: softmax statistics of head w over this split
    float mx = -__builtin_huge_valf();
    for (int i = lane; i < SPLIT; i += 64) mx = fmaxf(mx, ps[wave][i]);
    mx = warp_max(mx);
    float sum = 0.f;
    for (int i = lane; i < SPLIT; i += 64) {
      const float p = ps[wave][i] == -__builtin_huge_valf() ? 0.f : __expf(ps[wave][i] - mx);
      ps[wave][i] = p;
      sum += p;
    }
    sum = warp_sum(sum);
    if (lane == 0) { stat[wave][0] = mx; stat[wave][1] = sum; }
  }
  __syncthreads();
  {
    // thread: head wave, dims 2*lane, 2*lane + 1
    float o0 = 0.f, o1 = 0.f;
    for (int jj = j0; jj <= j1; ++jj) {
      const uint32_t vv = *(const uint32_t*)(kv_src(a.kv, a.kv.v, slot, jj, kvh, nkv) + 2 * lane);
      const float p = ps[wave][jj - j0];
      o0 = fmaf(p, h2f((f16_t)(vv & 0xffffu)), o0);
      o1 = fmaf(p, h2f((f16_t)(vv >> 16)), o1);
    }
    float* dst = part + (size_t)wave * head_stride;
    if (lane == 0) { dst[0] = stat[wave][0]; dst[1] = stat[wave][1]; }
    dst[2 + 2 * lane] = o0;
    dst[3 + 2 * lane] = o1;
  }
}

__global__ void __launch_bounds__(128) k_attn_merge(AttnArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int pos = a.rows.pos[r];
  const int k_lo = a.window > 0 ? max(0, pos - (a.window - 1)) : 0;
  const int ns = (pos - k_lo) / SPLIT + 1;
  const float* part = a.part + ((size_t)r * a.n_q_heads + h) * a.max_splits * (kHeadDim + 2);
  float mx = -__builtin_huge_valf();
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, part[(size_t)s * (kHeadDim + 2)]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* p = part + (size_t)s * (kHeadDim + 2);
    const float w = p[0] == -__builtin_huge_valf() ? 0.f : __expf(p[0] - mx);
    l = fmaf(w, p[1], l);
    o = fmaf(w, p[2 + d], o);
  }
  const float gate = sigmoidf_(a.gate[(size_t)r * a.ldg + h]);
  a.out[(size_t)r * a.n_q_heads * kHeadDim + (size_t)h * kHeadDim + d] = f2h(l > 0.f ? o / l * gate : 0.f);
}

hipError_t launch_attn_decode(hipStream_t s, const AttnArgs& a) {
  if (a.rows.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn_decode, dim3(a.max_splits, a.n_kv_heads, a.rows.n), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(a.rows.n, a.n_q_heads), dim3(kHeadDim), 0, s, a);
  return hipGetLastError();
}

}  // namespace lfm3
