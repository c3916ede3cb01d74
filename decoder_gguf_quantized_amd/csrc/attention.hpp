// Grouped-query attention over the f32 KV cache, decode (split over positions)
// and prefill (causal / sliding window), with an online softmax.
//
// Qwen3 walkthrough, Step 5 "The whole attention function": scores q.k scaled
// by head_dim^-1/2, causal mask, softmax, weighted sum of V, KV heads repeated
// over their query heads (query head h reads KV head h / (n_head / n_kv)).
// The online softmax (running max m, running sum l, rescaled accumulator) gives
// the same result as softmax-then-sum up to rounding.  Scores are kept in the
// log2 domain (q pre-scaled by head_dim^-1/2 * log2 e) so each exponential is
// one exp2.  Causal rule with a non-empty cache: the query at absolute position
// p sees keys j <= p; sliding-window layers also need j > p - window.
//
// Layout: a lane group of head_dim/8 lanes owns one position (decode) or one
// query (prefill); each lane holds 8 consecutive dims, so a group reads a K or V
// row as one contiguous, coalesced segment.  Dot products finish with a DPP
// tree inside the group.
#pragma once
#include "common.hpp"

namespace qd {

struct AttnDecodeArgs {
  const float* qkv;     // [B][ldqkv] raw projections q | k | v (before QK-norm and RoPE)
  int ldqkv;
  float* kc;            // layer base of the cache: [B][nkv][ctx][hd]
  float* vc;
  int ctx;
  const int* pos;       // [B] position of the new token
  int nq, nkv;
  int window;           // 0 = full causal
  int chunk;            // positions per workgroup
  int nchunk;
  const float* q_norm;  // [hd] or null (no QK-norm)
  const float* k_norm;
  float eps;
  const float2* rope;   // [ctx][hd/2] (cos, sin) of f32(pos) * inv_freq[i]
  float scale_log2;     // hd^-1/2 * log2(e)
  float* part_o;        // [B][nq][nchunk][hd], unnormalised partial outputs
  float* part_ml;       // [B][nq][nchunk][2]: running max (log2 domain), sum
  int* counter;         // [B][nkv] finished-chunk counters, zero between launches
  float* out;           // [B][nq*hd] merged attention output
};

// Device-coherent (write-through / L2-bypassing) accesses for the cross-
// workgroup partials: the L2s of the eight dies are not coherent with each
// other, and these keep the merge free of whole-cache write-back/invalidate.
QD_DEV void store_coherent(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
QD_DEV float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Most position chunks per (sequence, KV head); the launcher sizes chunks so.
constexpr int kMaxChunks = 64;

QD_DEV void attn_key_range(int p, int window, int& lo, int& hi) {
  hi = p;
  lo = window > 0 ? max(0, p - window + 1) : 0;
}

// Per-head RMSNorm (gain nw, or none) and the half-split rotation of one head
// held as 8 dims per lane over a group of LG = hd/8 lanes.  Dim d pairs with
// d + hd/2, which lives in lane li ^ (LG/2) at the same slot.
template <int LG>
QD_DEV void norm_rope_group(float (&v)[8], const float* nw, float eps, int hd, int li, const float (&c)[8],
                            const float (&sn)[8]) {
  if (nw) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    ss = group_sum<LG>(ss);
    const float scale = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * scale * nw[8 * li + e];
  }
  const bool first_half = li < LG / 2;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float other = __shfl_xor(v[e], LG / 2);
    v[e] = first_half ? v[e] * c[e] - other * sn[e] : v[e] * c[e] + other * sn[e];
  }
}

// Workgroup = (chunk of positions, KV head, sequence); it serves the KV head's
// whole group of query heads.  Prologue: QK-norm + RoPE of the group's queries,
// and, in the chunk that holds the new position, of the new key, which it also
// appends (with the new value) to the cache.  Each workgroup writes one partial
// (m, l, o) per query head; the workgroup that finishes last among the chunks
// of its (sequence, KV head) merges them (a counter, no workgroup waits):
//   O = sum_c o_c 2^(m_c - M) / sum_c l_c 2^(m_c - M),  M = max_c m_c.
template <int HD, int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnDecodeArgs a) {
  constexpr int LG = HD / 8;      // lanes per position
  constexpr int NG = 256 / LG;    // position streams per workgroup
  __shared__ float sm_o[NG][G][HD];
  __shared__ float sm_m[NG][G], sm_l[NG][G];
  __shared__ float sm_pm[G][kMaxChunks], sm_pl[G][kMaxChunks];
  __shared__ int sm_last;

  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int p = a.pos[s];
  int lo, hi;
  attn_key_range(p, a.window, lo, hi);
  const int c_lo = lo / a.chunk, c_hi = hi / a.chunk;
  if (c < c_lo || c > c_hi) return;
  const int start = max(lo, c * a.chunk), end = min(hi + 1, (c + 1) * a.chunk);

  const int tid = threadIdx.x, gi = tid / LG, li = tid % LG;
  const float* row = a.qkv + (size_t)s * a.ldqkv;
  float cs[8], sn[8];
  {
    const float2* rt = a.rope + (size_t)p * (HD / 2) + (8 * li) % (HD / 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 t = rt[e];
      cs[e] = t.x;
      sn[e] = t.y;
    }
  }
  float q[G][8], o[G][8], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4* qp = reinterpret_cast<const float4*>(row + (size_t)(g * G + h) * HD + li * 8);
    float4 q0 = qp[0], q1 = qp[1];
    float v[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    norm_rope_group<LG>(v, a.q_norm, a.eps, HD, li, cs, sn);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[h][e] = v[e] * a.scale_log2;
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  const size_t head_base = ((size_t)s * a.nkv + g) * a.ctx;
  float kn[8], vn[8];
  const bool has_new = c == c_hi;
  if (has_new) {
    const float4* kp = reinterpret_cast<const float4*>(row + (size_t)(a.nq + g) * HD + li * 8);
    const float4* vp = reinterpret_cast<const float4*>(row + (size_t)(a.nq + a.nkv + g) * HD + li * 8);
    float4 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
    float kv8[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    norm_rope_group<LG>(kv8, a.k_norm, a.eps, HD, li, cs, sn);
#pragma unroll
    for (int e = 0; e < 8; ++e) kn[e] = kv8[e];
    vn[0] = v0.x; vn[1] = v0.y; vn[2] = v0.z; vn[3] = v0.w;
    vn[4] = v1.x; vn[5] = v1.y; vn[6] = v1.z; vn[7] = v1.w;
    if (gi == 0) {
      float4* kd = reinterpret_cast<float4*>(a.kc + (head_base + p) * HD + li * 8);
      float4* vd = reinterpret_cast<float4*>(a.vc + (head_base + p) * HD + li * 8);
      kd[0] = make_float4(kn[0], kn[1], kn[2], kn[3]);
      kd[1] = make_float4(kn[4], kn[5], kn[6], kn[7]);
      vd[0] = v0;
      vd[1] = v1;
    }
  }
  // two positions per stream per iteration: both rows are requested before use
  auto fetch = [&](int j, float (&k)[8], float (&v)[8]) {
    if (has_new && j == p) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        k[e] = kn[e];
        v[e] = vn[e];
      }
    } else {
      const float4* kp = reinterpret_cast<const float4*>(a.kc + (head_base + j) * HD + li * 8);
      const float4* vp = reinterpret_cast<const float4*>(a.vc + (head_base + j) * HD + li * 8);
      const float4 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
      k[0] = k0.x; k[1] = k0.y; k[2] = k0.z; k[3] = k0.w; k[4] = k1.x; k[5] = k1.y; k[6] = k1.z; k[7] = k1.w;
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w; v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    }
  };
  auto accumulate = [&](const float (&k)[8], const float (&v)[8]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += q[h][e] * k[e];
      const float sc = group_sum<LG>(dot);
      const float mn = fmaxf(m[h], sc);
      const float corr = exp2f(m[h] - mn);
      const float pr = exp2f(sc - mn);
      l[h] = l[h] * corr + pr;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = o[h][e] * corr + pr * v[e];
      m[h] = mn;
    }
  };
  int j = start + gi;
  for (; j + NG < end; j += 2 * NG) {
    float k0[8], v0[8], k1[8], v1[8];
    fetch(j, k0, v0);
    fetch(j + NG, k1, v1);
    accumulate(k0, v0);
    accumulate(k1, v1);
  }
  if (j < end) {
    float k0[8], v0[8];
    fetch(j, k0, v0);
    accumulate(k0, v0);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[gi][h][li * 8 + e] = o[h][e];
    if (li == 0) {
      sm_m[gi][h] = m[h];
      sm_l[gi][h] = l[h];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * HD; idx += 256) {
    const int h = idx / HD, dd = idx % HD;
    float M = -INFINITY;
    for (int k = 0; k < NG; ++k) M = fmaxf(M, sm_m[k][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int k = 0; k < NG; ++k) {
        const float w = sm_m[k][h] == -INFINITY ? 0.f : exp2f(sm_m[k][h] - M);
        L += sm_l[k][h] * w;
        O += sm_o[k][h][dd] * w;
      }
    }
    const size_t pi = ((size_t)s * a.nq + g * G + h) * a.nchunk + c;
    store_coherent(a.part_o + pi * HD + dd, O);
    if (dd == 0) {
      store_coherent(a.part_ml + pi * 2 + 0, M);
      store_coherent(a.part_ml + pi * 2 + 1, L);
    }
  }
  // every partial store of this workgroup is complete before the counter moves
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int done = __hip_atomic_fetch_add(a.counter + s * a.nkv + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm_last = done == c_hi - c_lo;
  }
  __syncthreads();
  if (!sm_last) return;
  // merge: (m, l) of every chunk into LDS, then each output element requests its
  // values of all chunks at once (one round trip) and sums them in chunk order
  const int nact = c_hi - c_lo + 1;  // <= kMaxChunks (the launcher sizes chunks so)
  for (int i = tid; i < G * nact; i += 256) {
    const int h = i / nact, cc = i % nact;
    const size_t pi = ((size_t)s * a.nq + g * G + h) * a.nchunk + c_lo + cc;
    sm_pm[h][cc] = load_coherent(a.part_ml + pi * 2);
    sm_pl[h][cc] = load_coherent(a.part_ml + pi * 2 + 1);
  }
  __syncthreads();
  for (int idx = tid; idx < G * HD; idx += 256) {
    const int h = idx / HD, dd = idx % HD;
    const float* po = a.part_o + (((size_t)s * a.nq + g * G + h) * a.nchunk + c_lo) * HD + dd;
    float M = -INFINITY;
    for (int cc = 0; cc < nact; ++cc) M = fmaxf(M, sm_pm[h][cc]);
    float L = 0.f, O = 0.f;
    for (int c0 = 0; c0 < nact; c0 += 16) {  // 16 chunks' values requested per round trip
      float ov[16];
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) ov[cc] = c0 + cc < nact ? load_coherent(po + (size_t)(c0 + cc) * HD) : 0.f;
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) {
        if (c0 + cc < nact) {
          const float mc = sm_pm[h][c0 + cc];
          const float w = mc == -INFINITY ? 0.f : exp2f(mc - M);
          L += sm_pl[h][c0 + cc] * w;
          O += ov[cc] * w;
        }
      }
    }
    a.out[(size_t)s * a.nq * HD + (size_t)(g * G + h) * HD + dd] = O / L;
  }
  if (tid == 0) __hip_atomic_store(a.counter + s * a.nkv + g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct AttnPrefillArgs {
  const float* q;       // [T][nq*hd]
  const float* kc;      // cache of this (layer, sequence): [nkv][ctx][hd]
  const float* vc;
  int ctx, T, pos0, nq, nkv, window;
  float scale_log2;
  float* out;           // [T][nq*hd]
};

// Workgroup = (tile of 256/LG consecutive queries, one query head).  K/V tiles
// of KT keys are staged in LDS and shared by all queries of the tile.
template <int HD, int KT>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnPrefillArgs a) {
  constexpr int LG = HD / 8;
  constexpr int QT = 256 / LG;
  __shared__ float4 Ks[KT][HD / 4];
  __shared__ float4 Vs[KT][HD / 4];
  const int tid = threadIdx.x, gi = tid / LG, li = tid % LG;
  // signed copies: the window bound below goes negative for early tiles
  const int bx = (int)blockIdx.x, h = (int)blockIdx.y, g = h / (a.nq / a.nkv);
  const int t = bx * QT + gi;
  const bool active = t < a.T;
  const int p = a.pos0 + t;
  const int tlast = min(a.T, (bx + 1) * QT) - 1;
  const int kmax = a.pos0 + tlast;
  const int kmin = a.window > 0 ? max(0, a.pos0 + bx * QT - a.window + 1) : 0;

  float q[8], o[8], m = -INFINITY, l = 0.f;
  {
    const int tq = active ? t : 0;
    const float4* qp = reinterpret_cast<const float4*>(a.q + (size_t)tq * a.nq * HD + (size_t)h * HD + li * 8);
    float4 q0 = qp[0], q1 = qp[1];
    q[0] = q0.x * a.scale_log2; q[1] = q0.y * a.scale_log2; q[2] = q0.z * a.scale_log2; q[3] = q0.w * a.scale_log2;
    q[4] = q1.x * a.scale_log2; q[5] = q1.y * a.scale_log2; q[6] = q1.z * a.scale_log2; q[7] = q1.w * a.scale_log2;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  const float4* kbase = reinterpret_cast<const float4*>(a.kc + (size_t)g * a.ctx * HD);
  const float4* vbase = reinterpret_cast<const float4*>(a.vc + (size_t)g * a.ctx * HD);
  const int jlo = active ? (a.window > 0 ? max(0, p - a.window + 1) : 0) : 1;
  const int jhi = active ? p : 0;

  for (int j0 = kmin; j0 <= kmax; j0 += KT) {
    const int nk = min(KT, kmax - j0 + 1);
    __syncthreads();
    for (int i = tid; i < nk * (HD / 4); i += 256) {
      int kk = i / (HD / 4), dv = i % (HD / 4);
      Ks[kk][dv] = kbase[(size_t)(j0 + kk) * (HD / 4) + dv];
      Vs[kk][dv] = vbase[(size_t)(j0 + kk) * (HD / 4) + dv];
    }
    __syncthreads();
    const int a0 = max(jlo, j0), a1 = min(jhi, j0 + nk - 1);
    for (int j = a0; j <= a1; ++j) {
      const int kk = j - j0;
      float4 k0 = Ks[kk][li * 2], k1 = Ks[kk][li * 2 + 1];
      float dot = q[0] * k0.x + q[1] * k0.y + q[2] * k0.z + q[3] * k0.w +
                  q[4] * k1.x + q[5] * k1.y + q[6] * k1.z + q[7] * k1.w;
      float sc = group_sum<LG>(dot);
      float mn = fmaxf(m, sc);
      float corr = exp2f(m - mn);
      float pr = exp2f(sc - mn);
      l = l * corr + pr;
      float4 v0 = Vs[kk][li * 2], v1 = Vs[kk][li * 2 + 1];
      o[0] = o[0] * corr + pr * v0.x; o[1] = o[1] * corr + pr * v0.y;
      o[2] = o[2] * corr + pr * v0.z; o[3] = o[3] * corr + pr * v0.w;
      o[4] = o[4] * corr + pr * v1.x; o[5] = o[5] * corr + pr * v1.y;
      o[6] = o[6] * corr + pr * v1.z; o[7] = o[7] * corr + pr * v1.w;
      m = mn;
    }
  }
  if (active) {
    float inv = 1.0f / l;
    float4* op = reinterpret_cast<float4*>(a.out + (size_t)t * a.nq * HD + (size_t)h * HD + li * 8);
    op[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    op[1] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
  }
}

}  // namespace qd
