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
  const float* q;       // [B][nq*hd], after QK-norm and RoPE
  const float* kc;      // layer base of the cache: [B][nkv][ctx][hd]
  const float* vc;
  int ctx;
  const int* pos;       // [B] position of the newest token (already in the cache)
  int nq, nkv;
  int window;           // 0 = full causal
  int chunk;            // positions per workgroup
  float scale_log2;     // hd^-1/2 * log2(e)
  float* part_o;        // [B][nq][nchunk][hd], unnormalised
  float* part_ml;       // [B][nq][nchunk][2]: running max (log2 domain), sum
  int nchunk;
};

QD_DEV void attn_key_range(int p, int window, int& lo, int& hi) {
  hi = p;
  lo = window > 0 ? max(0, p - window + 1) : 0;
}

template <int HD, int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnDecodeArgs a) {
  constexpr int LG = HD / 8;      // lanes per position
  constexpr int NG = 256 / LG;    // position streams per workgroup
  __shared__ float sm_o[NG][G][HD];
  __shared__ float sm_m[NG][G], sm_l[NG][G];

  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int p = a.pos[s];
  int lo, hi;
  attn_key_range(p, a.window, lo, hi);
  const int c_lo = lo / a.chunk, c_hi = hi / a.chunk;
  if (c < c_lo || c > c_hi) return;
  const int start = max(lo, c * a.chunk), end = min(hi + 1, (c + 1) * a.chunk);

  const int tid = threadIdx.x, gi = tid / LG, li = tid % LG;
  const int group = a.nq / a.nkv;
  float q[G][8], o[G][8], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4* qp = reinterpret_cast<const float4*>(a.q + (size_t)s * a.nq * HD + (size_t)(g * group + h) * HD + li * 8);
    float4 q0 = qp[0], q1 = qp[1];
    q[h][0] = q0.x * a.scale_log2; q[h][1] = q0.y * a.scale_log2;
    q[h][2] = q0.z * a.scale_log2; q[h][3] = q0.w * a.scale_log2;
    q[h][4] = q1.x * a.scale_log2; q[h][5] = q1.y * a.scale_log2;
    q[h][6] = q1.z * a.scale_log2; q[h][7] = q1.w * a.scale_log2;
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  const size_t head_base = ((size_t)s * a.nkv + g) * a.ctx;
  for (int j = start + gi; j < end; j += NG) {
    const float4* kp = reinterpret_cast<const float4*>(a.kc + (head_base + j) * HD + li * 8);
    const float4* vp = reinterpret_cast<const float4*>(a.vc + (head_base + j) * HD + li * 8);
    float4 k0 = kp[0], k1 = kp[1];
    float4 v0 = vp[0], v1 = vp[1];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float dot = q[h][0] * k0.x + q[h][1] * k0.y + q[h][2] * k0.z + q[h][3] * k0.w +
                  q[h][4] * k1.x + q[h][5] * k1.y + q[h][6] * k1.z + q[h][7] * k1.w;
      float sc = group_sum<LG>(dot);
      float mn = fmaxf(m[h], sc);
      float corr = exp2f(m[h] - mn);
      float pr = exp2f(sc - mn);
      l[h] = l[h] * corr + pr;
      o[h][0] = o[h][0] * corr + pr * v0.x; o[h][1] = o[h][1] * corr + pr * v0.y;
      o[h][2] = o[h][2] * corr + pr * v0.z; o[h][3] = o[h][3] * corr + pr * v0.w;
      o[h][4] = o[h][4] * corr + pr * v1.x; o[h][5] = o[h][5] * corr + pr * v1.y;
      o[h][6] = o[h][6] * corr + pr * v1.z; o[h][7] = o[h][7] * corr + pr * v1.w;
      m[h] = mn;
    }
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
        float w = sm_m[k][h] == -INFINITY ? 0.f : exp2f(sm_m[k][h] - M);
        L += sm_l[k][h] * w;
        O += sm_o[k][h][dd] * w;
      }
    }
    const size_t pi = ((size_t)s * a.nq + g * group + h) * a.nchunk + c;
    a.part_o[pi * HD + dd] = O;
    if (dd == 0) {
      a.part_ml[pi * 2 + 0] = M;
      a.part_ml[pi * 2 + 1] = L;
    }
  }
}

struct AttnCombineArgs {
  const float* part_o;
  const float* part_ml;
  const int* pos;
  int nq, hd, window, chunk, nchunk;
  float* out;           // [B][nq*hd]
};

// One workgroup per (query head, sequence); thread dd merges dimension dd over
// the chunks that hold keys: O = sum_c o_c 2^(m_c - M) / sum_c l_c 2^(m_c - M).
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnCombineArgs a) {
  const int h = blockIdx.x, s = blockIdx.y, dd = threadIdx.x;
  if (dd >= a.hd) return;
  int lo, hi;
  attn_key_range(a.pos[s], a.window, lo, hi);
  const int c_lo = lo / a.chunk, c_hi = hi / a.chunk;
  const size_t base = ((size_t)s * a.nq + h) * a.nchunk;
  float M = -INFINITY;
  for (int c = c_lo; c <= c_hi; ++c) M = fmaxf(M, a.part_ml[(base + c) * 2]);
  float L = 0.f, O = 0.f;
  for (int c = c_lo; c <= c_hi; ++c) {
    float mc = a.part_ml[(base + c) * 2];
    float w = mc == -INFINITY ? 0.f : exp2f(mc - M);
    L += a.part_ml[(base + c) * 2 + 1] * w;
    O += a.part_o[(base + c) * a.hd + dd] * w;
  }
  a.out[(size_t)s * a.nq * a.hd + (size_t)h * a.hd + dd] = O / L;
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
