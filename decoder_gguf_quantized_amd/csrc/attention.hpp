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
// Decode: a lane group of head_dim/8 lanes owns one position; each lane holds
// 8 of its dims, so a group reads a K or V row as contiguous, coalesced
// segments, and dot products finish with a DPP tree inside the group.
// Prefill: 32 queries x 32 keys per tile on the matrix cores (layouts at the
// kernels below).
#pragma once
#include <type_traits>

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
  const float2* rope;   // [B][hd/2] (cos, sin) of f32(pos[s]) * inv_freq[i]: each sequence's
                        // row of the layer's RoPE table, copied at step start
  float scale_log2;     // hd^-1/2 * log2(e)
  float* acc;           // this layer's accumulators: kAccCopies blocks of o [rows][nq][hd]
                        // then l [rows][nq] (zero on entry); chunk c adds into block
                        // c % kAccCopies
  float* acc_clear;     // the other layer parity's accumulators, zeroed here for the next layer
  int acc_rows;         // rows (max_seqs) of each accumulator block
  int* err;             // host-mapped error word (2: a chunk's scores beyond the merge's range)
  const int* seq;       // [B] sequence slot of each row, or null (row b is sequence b)
  KvMap map;            // cache layout (the paged kernel reads map.table)
  int gsplit;           // workgroups per KV head (1, or 2: eight query heads per KV head run as
                        // two groups of four, each streaming the head's cache; a group of eight
                        // holds more registers than the SIMD has and spills)
};

// Most position chunks per (sequence, KV head); the launcher sizes chunks so
// (it bounds the grid at long contexts).
constexpr int kMaxChunks = 64;

QD_DEV void attn_key_range(int p, int window, int& lo, int& hi) {
  hi = p;
  lo = window > 0 ? max(0, p - window + 1) : 0;
}

// Per-head RMSNorm (gain nw, or none) and the half-split rotation of one head
// held over a group of LG = hd/8 lanes: lane li holds dims 4 li + e (v[e]) and
// hd/2 + 4 li + e (v[4 + e]), e < 4, so each rotation pair (d, d + hd/2) sits in
// one lane and c/sn hold the lane's four angles.
template <int LG>
QD_DEV void norm_rope_group(float (&v)[8], bool norm, const float (&nw)[8], float eps, int hd, const float (&c)[4],
                            const float (&sn)[4]) {
  if (norm) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    ss = group_sum<LG>(ss);
    const float scale = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * scale * nw[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x1 = v[e], x2 = v[4 + e];
    v[e] = x1 * c[e] - x2 * sn[e];
    v[4 + e] = x2 * c[e] + x1 * sn[e];
  }
}

// The lane's 8 values of a head row in the lane layout above: two float4
// loads, each covering 16 consecutive bytes per lane (256 contiguous bytes over
// a 16-lane group at hd = 128).
QD_DEV void load_lane8(const float* rowp, int hd, int li, float (&v)[8]) {
  const float4* p = reinterpret_cast<const float4*>(rowp);
  const float4 a = p[li], b = p[hd / 8 + li];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Same, with non-temporal loads (cache rows are streamed once per step).
QD_DEV void load_lane8_nt(const float* rowp, int hd, int li, float (&v)[8]) {
  const float4* p = reinterpret_cast<const float4*>(rowp);
  const float4 a = load_nt(p + li), b = load_nt(p + hd / 8 + li);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

QD_DEV void store_lane8(float* rowp, int hd, int li, const float (&v)[8]) {
  float4* p = reinterpret_cast<float4*>(rowp);
  p[li] = make_float4(v[0], v[1], v[2], v[3]);
  p[hd / 8 + li] = make_float4(v[4], v[5], v[6], v[7]);
}

// Workgroup = (chunk of positions, KV head, sequence); it serves the KV head's
// whole group of query heads.  Prologue: QK-norm + RoPE of the group's queries
// and of the new key; the chunk that holds the new position also appends the
// new key and value to the cache.
//
// Merge without a second round trip.  A split softmax needs a common reference
// for the chunks' maxima.  Every workgroup can compute the same one without
// communicating: the new token's own score R_h = q_h . k_new (every query sees
// its own key, on every layer, windowed or not), evaluated by every workgroup
// with the same operations on the same registers, so the values agree bit for
// bit.  A workgroup reduces its streams to (M, L, O) per head, rescales them
// to R_h by f = 2^(M - R_h) and adds f L and f O into f32 accumulators with
// hardware atomic adds: no counter, no wait, no last-workgroup merge (which
// cost about 4.5 us of the 8B-shape layer's 11.9 us: store acknowledgements,
// the counter's round trip, the merging workgroup's loads).  Chunks alternate
// between two accumulator blocks: adds to one address are serialised in the
// memory system, and two blocks halve that chain.  The consumer (the O
// projection's input staging) sums the blocks and divides:
//   o_h = sum_c f_c O_c / sum_c f_c L_c,
// the softmax-weighted sum of the values, as with any common reference.  The
// new key's own term has weight 2^0 = 1, so the denominator is at least 1; a
// chunk whose maximum lies 100 or more log2 units above R_h (or whose scores
// are NaN) would leave f32's range, so it latches *err = 2 (the next call
// reports it) instead.  The adds are f32 and their order varies from run to
// run, so decode results agree to f32 rounding, not bit for bit.
// The accumulators of the two layer parities alternate: this launch zeroes
// the other parity's blocks, which the previous layer's O projection has
// finished reading and the next layer's attention adds into.
//
// Latency: the kernel is a short chain of dependent memory round trips, so
// every request that does not need the new position goes out before it
// arrives: the RoPE row (copied per sequence at step start), the raw queries
// and new key/value, and on full-causal layers the chunk's first keys and
// values (a chunk's addresses do not depend on the position; keys past it are
// masked).  The walk takes two position pairs per stream per round.
// PAGED: the cache is paged; a chunk lies in one page (the host keeps chunks
// no longer than a page), so one table entry per workgroup places all of it.
template <int HD, int G, bool PAGED>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnDecodeArgs a) {
  constexpr int LG = HD / 8;      // lanes per position
  constexpr int NG = 256 / LG;    // position streams per workgroup
  // each wave's streams merged to one (M, L, O) per head (stream_reduce)
  __shared__ float sm_o[4][G][HD];
  __shared__ float sm_m[4][G], sm_l[4][G];

  // g: the workgroup's group of G query heads (heads g G .. g G + G - 1), kvh
  // their KV head
  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z, kvh = g / a.gsplit;
  const int tid = threadIdx.x, gi = tid / LG, li = tid % LG;
  const float* row = a.qkv + (size_t)s * a.ldqkv;
  const int sq = a.seq ? a.seq[s] : s;
  const int cb = c * a.chunk;
  // cache row of position j is head_base + (j & pmask) for every j of this
  // chunk (pmask: a window layer's ring, else all ones)
  size_t head_base;
  int pmask = -1;
  if constexpr (PAGED) {
    const int pi = cb >> a.map.log2p;
    const int pg = a.map.table[sq * a.map.tw + pi];
    head_base = (((size_t)pg * a.nkv + kvh) << a.map.log2p) - ((size_t)pi << a.map.log2p);
  } else if (a.map.ring) {
    head_base = ((size_t)sq * a.nkv + kvh) << a.map.ring;
    pmask = (1 << a.map.ring) - 1;
  } else {
    head_base = ((size_t)sq * a.nkv + kvh) * a.ctx;
  }
  const bool spec = a.window == 0;

  const int p = a.pos[s];
  // lane li of a stream group holds dims 4 li + e and HD/2 + 4 li + e (e < 4)
  float cs[4], sn[4];
  {
    const float2* rt = a.rope + (size_t)s * (HD / 2) + 4 * li;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 t = rt[e];
      cs[e] = t.x;
      sn[e] = t.y;
    }
  }
  float q[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) load_lane8(row + (size_t)(g * G + h) * HD, HD, li, q[h]);
  // the lane's 8 dims of the QK-norm gains, requested with the rest (without
  // a norm the row itself stands in, unused: every path issues the same loads,
  // so that each wait below is for exactly the data it needs)
  const bool qkn = a.q_norm != nullptr;
  float wq[8], wk[8];
  load_lane8(qkn ? a.q_norm : row, HD, li, wq);
  load_lane8(qkn ? a.k_norm : row, HD, li, wk);
  float kn[8], vn[8];
  load_lane8(row + (size_t)(a.nq + kvh) * HD, HD, li, kn);
  load_lane8(row + (size_t)(a.nq + a.nkv + kvh) * HD, HD, li, vn);
  // keys/values of positions j0 and j0 + NG (addresses clamped into the cache;
  // positions outside [start, end) are masked when accumulated)
  auto fetch_pair = [&](int j0, float (&k)[2][8], float (&v)[2][8]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int jj = min(j0 + t * NG, a.ctx - 1);
      load_lane8_nt(a.kc + (head_base + (jj & pmask)) * HD, HD, li, k[t]);
      load_lane8_nt(a.vc + (head_base + (jj & pmask)) * HD, HD, li, v[t]);
    }
  };
  float ka[2][8], va[2][8], kb[2][8], vb[2][8];
  // the chunk's first two pairs (four positions per stream), requested before
  // the new position arrives: their addresses do not depend on it.  They go
  // out after the loads above (the scheduler may not move loads across this
  // point): loads return in order, and the queries must not wait for the cache.
  __builtin_amdgcn_sched_barrier(0);
  fetch_pair(cb + gi, ka, va);
  fetch_pair(cb + 2 * NG + gi, kb, vb);

  // The other parity's accumulators are zeroed by all workgroups together;
  // workgroups with work do their share after their last load (loads and
  // stores share one in-order counter: a store in flight would turn every
  // wait for a load into a wait for all of them).
  auto clear_other = [&] {
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    const int wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const size_t n = (size_t)kAccCopies * a.acc_rows * a.nq * (HD + 1);
    for (size_t i = (size_t)wg * 256 + tid; i < n; i += (size_t)nwg * 256) a.acc_clear[i] = 0.f;
  };

  int lo, hi;
  attn_key_range(p, a.window, lo, hi);
  const int c_lo = lo / a.chunk, c_hi = hi / a.chunk;
  if (c < c_lo || c > c_hi) {
    clear_other();
    return;
  }
  const int start = max(lo, cb), end = min(hi + 1, cb + a.chunk);
  // first position pair of the chunk's walk (windowed layers skip whole pairs
  // below the window)
  const int jb0 = spec ? cb : cb + ((start - cb) / (2 * NG)) * (2 * NG);
  if (jb0 != cb) {  // a windowed layer whose walk starts further in
    fetch_pair(jb0 + gi, ka, va);
    fetch_pair(jb0 + 2 * NG + gi, kb, vb);
  }

  float o[G][8], m[G], l[G], ref[G];
  norm_rope_group<LG>(kn, qkn, wk, a.eps, HD, cs, sn);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    norm_rope_group<LG>(q[h], qkn, wq, a.eps, HD, cs, sn);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q[h][e] *= a.scale_log2;
      o[h][e] = 0.f;
    }
    m[h] = -INFINITY;
    l[h] = 0.f;
    // the merge reference: the new key's score (the same expression as its
    // score in the walk below)
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += q[h][e] * kn[e];
    ref[h] = group_sum<LG>(dot);
  }
  const bool has_new = c == c_hi;
  // online softmax over the two positions of a pair (j0, j0 + NG): one
  // rescale of the state per pair.  Masked positions take no part (selects, no
  // branch: every lane of a stream group takes the same path).  A masked
  // position's row may never have been written (cache rows past the new
  // position are requested ahead), so its values are replaced by zeros before
  // any arithmetic: 0 * NaN would otherwise reach the output.
  auto accumulate = [&](int j0, const float (&kc)[2][8], const float (&vc)[2][8]) {
    bool valid[2];
    float k[2][8], v[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = j0 + t * NG;
      valid[t] = j >= start && j < end;
      const bool is_new = has_new && j == p;  // its cache row is written at the end: use the registers
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        k[t][e] = is_new ? kn[e] : (valid[t] ? kc[t][e] : 0.f);
        v[t][e] = is_new ? vn[e] : (valid[t] ? vc[t][e] : 0.f);
      }
    }
    const bool any = valid[0] || valid[1];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += q[h][e] * k[t][e];
        sc[t] = group_sum<LG>(dot);
      }
      const float mn = any ? fmaxf(m[h], fmaxf(valid[0] ? sc[0] : -INFINITY, valid[1] ? sc[1] : -INFINITY)) : m[h];
      const float corr = any ? exp2f(m[h] - mn) : 1.f;
      const float p0 = valid[0] ? exp2f(sc[0] - mn) : 0.f;
      const float p1 = valid[1] ? exp2f(sc[1] - mn) : 0.f;
      l[h] = l[h] * corr + (p0 + p1);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = o[h][e] * corr + (p0 * v[0][e] + p1 * v[1][e]);
      m[h] = mn;
    }
  };
  // walk of the chunk two pairs at a time (wave-uniform trip count: jb and end
  // are the same for every lane); both pairs are in flight when a round
  // starts, and the loads of a round are issued on every path that reaches it
  for (int jb = jb0;; jb += 4 * NG) {
    accumulate(jb + gi, ka, va);
    accumulate(jb + 2 * NG + gi, kb, vb);
    if (jb + 4 * NG >= end) break;
    fetch_pair(jb + 4 * NG + gi, ka, va);
    fetch_pair(jb + 6 * NG + gi, kb, vb);
  }
  // Merge the streams.  Inside a wave (64 / LG streams, lanes l and l + LG k
  // hold the same dims) the maxima, weights and sums move between lane rows
  // with cross-lane swaps (no LDS); then one (M, L, O) per wave and head goes
  // through LDS, the workgroup's four are merged, rescaled to the reference and
  // added to the accumulators.
  const int wave = tid >> 6;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = stream_reduce<LG, true>(m[h]);
    const float w = m[h] == -INFINITY ? 0.f : exp2f(m[h] - M);
    const float L = stream_reduce<LG, false>(w * l[h]);
    float ow[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ow[e] = stream_reduce<LG, false>(w * o[h][e]);
    if (gi % (64 / LG) == 0) {  // the wave's first stream writes the merged values
      store_lane8(&sm_o[wave][h][0], HD, li, ow);
      if (li == 0) {
        sm_m[wave][h] = M;
        sm_l[wave][h] = L;
      }
    }
  }
  __syncthreads();
  // every load of the kernel has been waited for: now the stores (the new key
  // and value into the cache, for the next steps; the other parity's clear)
  if (has_new && gi == 0 && g % a.gsplit == 0) {  // one writer per KV head
    store_lane8(a.kc + (head_base + (p & pmask)) * HD, HD, li, kn);
    store_lane8(a.vc + (head_base + (p & pmask)) * HD, HD, li, vn);
  }
  clear_other();
  float* acc_blk = a.acc + (size_t)(c % kAccCopies) * ((size_t)a.acc_rows * a.nq * (HD + 1));
  float* acc_o = acc_blk + ((size_t)s * a.nq + g * G) * HD;
  float* acc_l = acc_blk + (size_t)a.acc_rows * a.nq * HD + (size_t)s * a.nq + g * G;
  for (int idx = tid; idx < G * HD; idx += 256) {
    const int h = idx / HD, dd = idx % HD;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][h]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_m[w][h];
      const float ww = mw == -INFINITY ? 0.f : exp2f(mw - M);
      O += ww * sm_o[w][h][dd];
      L += ww * sm_l[w][h];
    }
    float rh = ref[0];  // ref[h] without a dynamic register index
#pragma unroll
    for (int t = 1; t < G; ++t) rh = t == h ? ref[t] : rh;
    float d = M - rh;
    if (!(d < 100.f)) {  // beyond f32's exponent range (or NaN scores): report, add nothing
      if (dd == 0 && a.err) *a.err = 2;
      d = -INFINITY;
    }
    const float f = exp2f(d);
    if (dd == 0) unsafeAtomicAdd(acc_l + h, L * f);
    unsafeAtomicAdd(acc_o + idx, O * f);
  }
}

struct AttnPrefillArgs {
  const float* q;       // [T][nq*hd]
  const float* kc;      // cache of this layer (rows placed by map)
  const float* vc;
  int ctx, T, pos0, nq, nkv, window;
  float scale_log2;
  float* out;           // [T][nq*hd]
  int seq;
  KvMap map;
};

// ------------------------------------------------------------ prefill attention on the matrix cores
// The online softmax of the decode kernel for T queries at once, with both
// products on V_MFMA_F32_32X32X2_F32 (f32 operands, f32 accumulation); head_dim
// 64 and 128.  Workgroup = 32 queries x one query head; its four waves take the
// 32-key tiles of the queries' key range in turn and merge their (max, sum,
// output) at the end.  Query tiles are dispatched last first, so the longest
// key ranges start first.
//
// Per tile the wave computes S^T = K Q^T (keys as rows, queries as columns),
// contracting over dims in the order c(t, h) = h * HD/2 + t (lane half h,
// step t), so each lane streams half of its key's row and keeps half of its
// query's row in registers.  The D layout of S^T puts query j in lanes j and
// j + 32 and keys 8(r/4) + 4h + r%4 in register r of lane half h; taking the
// P V contraction over keys in exactly that order, register t of P^T is the B
// operand of step t of O^T = V^T P^T, so the probabilities never move.  Row i
// of output block b is dim NB i + b (NB = HD / 32 blocks), so the A operands a
// lane needs from one value row, one per block, are NB consecutive floats: one
// vector load per key.  Scores are in the log2 domain (q scaled by
// log2(e)/sqrt(hd)); masked keys get probability 0.
//
// Two workgroups per CU (two waves per SIMD): the queries, scaled, sit in LDS
// (read four dims at a time per step group) rather than in registers, so a
// wave fits in 256 registers and one wave's loads, softmax and merges overlap
// the other's matrix products.  A tile's values are requested together with
// its keys, before the scores (which they do not depend on).  A 32-aligned
// tile lies in one page of a paged cache (pages hold at least 32 positions),
// so one table entry places all of its rows.
template <int HD>
__global__ __launch_bounds__(256, 2) void attn_prefill_mfma_kernel(AttnPrefillArgs a) {
  static_assert(HD == 64 || HD == 128, "whole-head kernel: head_dim 64 or 128");
  constexpr int HH = HD / 2;  // contraction steps of S^T (two dims per step)
  constexpr int NB = HD / 32; // 32-dim blocks of the output
  constexpr int QS = HD + 4;  // LDS row stride of the queries (bank spread for row-per-lane reads)
  typedef float vnb __attribute__((ext_vector_type(NB)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  // the queries during the walk, then the waves' partial results for the merge
  __shared__ float sm_raw[3 * NB * 16 * 64 + 3 * 2 * 64 > 32 * QS ? 3 * NB * 16 * 64 + 3 * 2 * 64 : 32 * QS];
  float (*q_s)[QS] = reinterpret_cast<float (*)[QS]>(sm_raw);
  float (*sm_o)[NB][16][64] = reinterpret_cast<float (*)[NB][16][64]>(sm_raw);
  float (*sm_ml)[2][64] = reinterpret_cast<float (*)[2][64]>(sm_raw + 3 * NB * 16 * 64);
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, lk = lane >> 5;
  // wave index as a uniform value, so tile addresses (and a page-table
  // lookup) are scalar work
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroup id -> (KV head, query head, query tile): consecutive ids take
  // consecutive KV heads, so with 8 KV heads (the XCD count) every workgroup of
  // a KV head runs on one XCD and its keys and values stay in that XCD's L2;
  // query tiles go last first, so the longest key ranges start first.
  const int G = a.nq / a.nkv, nqt = (int)gridDim.x / a.nq;
  const int g = (int)blockIdx.x % a.nkv, rest = (int)blockIdx.x / a.nkv;
  const int h = g * G + rest % G, q0 = (nqt - 1 - rest / G) * 32;
  const int tq = q0 + li;  // this lane's query (token index)
  const bool q_ok = tq < a.T;
  const int p = a.pos0 + tq;
  const int tlast = min(a.T, q0 + 32) - 1;
  const int kmax = a.pos0 + tlast;
  const int kmin = a.window > 0 ? max(0, a.pos0 + q0 - a.window + 1) : 0;
  const int kt0 = kmin & ~31;
  const int ntile = (kmax - kt0) / 32 + 1;
  // the lane's query sees keys [k_lo, k_hi] (none past the prompt's end)
  const int k_hi = q_ok ? p : -1, k_lo = a.window > 0 ? p - a.window + 1 : 0;

  // the 32 queries of head h, scaled, into LDS (rows past the prompt read row 0)
  for (int i = tid; i < 32 * HD / 4; i += 256) {
    const int r = i / (HD / 4), c4 = i % (HD / 4);
    const int t = q0 + r < a.T ? q0 + r : 0;
    const float4 v = *reinterpret_cast<const float4*>(a.q + (size_t)t * a.nq * HD + (size_t)h * HD + 4 * c4);
    *reinterpret_cast<float4*>(&q_s[r][4 * c4]) =
        make_float4(v.x * a.scale_log2, v.y * a.scale_log2, v.z * a.scale_log2, v.w * a.scale_log2);
  }
  f32x16 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // Tile rows are read through a buffer descriptor that starts at the tile's
  // first row and ends after row kmax: rows past it read as zeros (finite, and
  // masked), and every address is a per-lane constant plus an immediate.
  // keys: lane (li, lk) reads K[key0 + li][lk * HH ...]; values: step t of
  // O^T = V^T P^T contracts keys 8(t/4) + 4h + t%4 (lane half h), the NB dims
  // NB li .. NB li + NB - 1 of each
  const int k_off = (li * HD + lk * HH) * 4;
  const int v_off = ((4 * lk) * HD + NB * li) * 4;
  // tiles that no query of the workgroup sees only in part skip the mask
  const int p_first = a.pos0 + q0, p_last = a.pos0 + tlast;
  __syncthreads();

  for (int it = wave; it < ntile; it += 4) {
    const int key0 = kt0 + 32 * it;
    const size_t base = kv_row(a.map, a.nkv, a.ctx, a.seq, g, key0);  // row of key0 + x is base + x
    const int bytes = (min(kmax - key0, 31) + 1) * HD * 4;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.kc + base * HD), (short)0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.vc + base * HD), (short)0, bytes, 0x00020000);
    u32x4 kb[HH / 4];
#pragma unroll
    for (int e = 0; e < HH / 4; ++e) kb[e] = __builtin_amdgcn_raw_buffer_load_b128(kr, k_off + 16 * e, 0, 0);
    vnb vb[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int off = v_off + (8 * (t >> 2) + (t & 3)) * HD * 4;
      if constexpr (NB == 4) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
        vb[t] = vnb{__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w)};
      } else {
        const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(vr, off, 0, 0);
        vb[t] = vnb{__uint_as_float(w.x), __uint_as_float(w.y)};
      }
    }
    // S^T = K Q^T (the queries are read from LDS on every tile: an opaque zero
    // in the address keeps the compiler from hoisting them into registers)
    int qz;
    asm volatile("s_mov_b32 %0, 0" : "=s"(qz));
    const float* qrow = &q_s[li][lk * HH + qz];
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int e = 0; e < HH / 4; ++e) {
      const float4 qv = *reinterpret_cast<const float4*>(qrow + 4 * e);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(kb[e].x), qv.x, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(kb[e].y), qv.y, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(kb[e].z), qv.z, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(kb[e].w), qv.w, sacc, 0, 0, 0);
    }
    // online softmax of query li over the tile's keys (16 here, 16 in lane ^ 32)
    const bool inner = key0 + 31 <= p_first && (a.window == 0 || key0 > p_last - a.window);
    if (!inner) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * lk + (r & 3);
        sacc[r] = ((key >= k_lo) & (key <= k_hi)) ? sacc[r] : -INFINITY;
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // lazy rescale: the reference max moves only when a score exceeds it by
    // more than 8 (probabilities stay below 2^8, exact in f32 either way), so
    // the output accumulators are rescaled on few tiles, and only when some
    // lane of the wave needs it.  A query with no key seen yet keeps -inf and
    // probabilities 0.
    const bool first = m_run == -INFINITY;
    const bool bump = !first && mt > m_run + 8.f;
    const float corr = bump ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
    m_run = first || bump ? mt : m_run;
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    float pr[16], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(sacc[r] - mref);  // exp2(-inf) = 0 for masked keys
      ps += pr[r];
    }
    ps += __shfl_xor(ps, 32);
    l_run = l_run * corr + ps;
    // O^T += V^T P^T
    if (__any(corr != 1.f)) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] *= corr;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(vb[t][b], pr[t], o[b], 0, 0, 0);
  }
  // merge the four waves' partial results into wave 0 (the LDS held the
  // queries until every wave's last product)
  __syncthreads();
  if (wave > 0) {
    sm_ml[wave - 1][0][lane] = m_run;
    sm_ml[wave - 1][1][lane] = l_run;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) sm_o[wave - 1][b][r][lane] = o[b][r];
  }
  __syncthreads();
  if (wave > 0 || !q_ok) return;
  float M = m_run;
#pragma unroll
  for (int w = 0; w < 3; ++w) M = fmaxf(M, sm_ml[w][0][lane]);
  const float w0 = M == -INFINITY ? 0.f : exp2f(m_run - M);
  float L = l_run * w0;
  float ww[3];
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    ww[w] = M == -INFINITY ? 0.f : exp2f(sm_ml[w][0][lane] - M);
    L += ww[w] * sm_ml[w][1][lane];
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  float* orow = a.out + (size_t)tq * a.nq * HD + (size_t)h * HD;
  // register r holds MFMA row i = 8(r/4) + 4 lk + r%4 of every block: dims NB i .. NB i + NB - 1
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    vnb v;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float acc = o[b][r] * w0;
#pragma unroll
      for (int w = 0; w < 3; ++w) acc += ww[w] * sm_o[w][b][r][lane];
      v[b] = acc * inv;
    }
    *reinterpret_cast<vnb*>(orow + NB * (8 * (r >> 2) + 4 * lk + (r & 3))) = v;
  }
}

// ------------------------------------------------------------ prefill attention, head-dim split
// head_dim 256 (at 128 the whole-head kernel above measured faster).  Same
// workgroup (32 queries x one query head), the same MFMA layouts and the same
// tile loads (buffer descriptors ending after the last key, the mask on edge
// tiles only, workgroup order) as attn_prefill_mfma_kernel, but the four waves
// walk every key tile together, each owning a quarter of the head dimension:
// wave w contracts dims [w HD/4, (w+1) HD/4) of S^T = K Q^T (contraction
// order c(t, h) = w HD/4 + h HD/8 + t), the four partial score tiles are
// summed through LDS in wave order (so every wave holds the same scores,
// maximum and sum), and wave w accumulates output dims [w HD/4, (w+1) HD/4)
// of O^T = V^T P^T (row i of its block b: dim w HD/4 + NBW i + b).  A wave
// then needs a quarter of the query, output, key and value registers of the
// whole-head kernel, which leaves room to request the next tile's keys and
// values while the current tile is multiplied; no merge of partial outputs is
// needed at the end.
template <int HD>
__global__ __launch_bounds__(256) void attn_prefill_dsplit_kernel(AttnPrefillArgs a) {
  static_assert(HD % 128 == 0, "a wave owns whole 32-dim output blocks");
  constexpr int D = HD / 4;     // dims owned by a wave
  constexpr int DH = D / 2;     // contraction steps of the wave's partial S^T
  constexpr int NBW = D / 32;   // 32-dim output blocks of the wave
  typedef float vnb __attribute__((ext_vector_type(NBW)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int uvnb __attribute__((ext_vector_type(NBW)));
  __shared__ float sm_s[2][4][16][64];  // partial S^T per wave, double-buffered by tile parity
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, lk = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup id -> (KV head, query head, query tile) as in attn_prefill_mfma_kernel
  const int G = a.nq / a.nkv, nqt = (int)gridDim.x / a.nq;
  const int g = (int)blockIdx.x % a.nkv, rest = (int)blockIdx.x / a.nkv;
  const int h = g * G + rest % G, q0 = (nqt - 1 - rest / G) * 32;
  const int tq = q0 + li;  // this lane's query (token index)
  const bool q_ok = tq < a.T;
  const int p = a.pos0 + tq;
  const int tlast = min(a.T, q0 + 32) - 1;
  const int kmax = a.pos0 + tlast;
  const int kmin = a.window > 0 ? max(0, a.pos0 + q0 - a.window + 1) : 0;
  const int kt0 = kmin & ~31;
  const int ntile = (kmax - kt0) / 32 + 1;
  const int dk = wave * D + lk * DH;  // first contraction dim of this lane
  const int k_hi = q_ok ? p : -1, k_lo = a.window > 0 ? p - a.window + 1 : 0;
  const int p_first = a.pos0 + q0, p_last = a.pos0 + tlast;

  float q[DH];
  {
    const float4* qp =
        reinterpret_cast<const float4*>(a.q + (size_t)(q_ok ? tq : 0) * a.nq * HD + (size_t)h * HD + dk);
#pragma unroll
    for (int e = 0; e < DH / 4; ++e) {
      const float4 v = qp[e];
      q[4 * e + 0] = v.x * a.scale_log2;
      q[4 * e + 1] = v.y * a.scale_log2;
      q[4 * e + 2] = v.z * a.scale_log2;
      q[4 * e + 3] = v.w * a.scale_log2;
    }
  }

  // one tile's operands: K[key0 + li][dk .. dk + DH) and, for O^T step t,
  // V[key0 + 8(t/4) + 4 lk + t%4][w D + NBW li .. + NBW), through descriptors
  // that end after row kmax (rows past it read as zeros)
  struct Tile {
    u32x4 k[DH / 4];
    vnb v[16];
  };
  const int k_off = (li * HD + dk) * 4;
  const int v_off = (4 * lk * HD + wave * D + NBW * li) * 4;
  auto load = [&](Tile& b, int it) {
    const int key0 = kt0 + 32 * it;
    const size_t base = kv_row(a.map, a.nkv, a.ctx, a.seq, g, key0);  // row of key0 + x is base + x
    const int bytes = (min(kmax - key0, 31) + 1) * HD * 4;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.kc + base * HD), (short)0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.vc + base * HD), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int e = 0; e < DH / 4; ++e) b.k[e] = __builtin_amdgcn_raw_buffer_load_b128(kr, k_off + 16 * e, 0, 0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int off = v_off + (8 * (t >> 2) + (t & 3)) * HD * 4;
      uvnb w;
      if constexpr (NBW == 2) w = __builtin_amdgcn_raw_buffer_load_b64(vr, off, 0, 0);
      else w = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
#pragma unroll
      for (int bb = 0; bb < NBW; ++bb) b.v[t][bb] = __uint_as_float(w[bb]);
    }
  };

  f32x16 o[NBW];
#pragma unroll
  for (int bb = 0; bb < NBW; ++bb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[bb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](const Tile& b, int it) {
    const int key0 = kt0 + 32 * it;
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int e = 0; e < DH / 4; ++e) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b.k[e].x), q[4 * e + 0], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b.k[e].y), q[4 * e + 1], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b.k[e].z), q[4 * e + 2], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b.k[e].w), q[4 * e + 3], sacc, 0, 0, 0);
    }
    // the whole-head scores: partial tiles summed in wave order
#pragma unroll
    for (int r = 0; r < 16; ++r) sm_s[it & 1][wave][r][lane] = sacc[r];
    __syncthreads();
    float sc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      sc[r] = ((sm_s[it & 1][0][r][lane] + sm_s[it & 1][1][r][lane]) + sm_s[it & 1][2][r][lane]) +
              sm_s[it & 1][3][r][lane];
    // tiles that no query of the workgroup sees only in part skip the mask
    const bool inner = key0 + 31 <= p_first && (a.window == 0 || key0 > p_last - a.window);
    if (!inner) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * lk + (r & 3);
        sc[r] = ((key >= k_lo) & (key <= k_hi)) ? sc[r] : -INFINITY;
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // lazy rescale, as in attn_prefill_mfma_kernel (every wave takes the same
    // decisions: its scores are the same)
    const bool first = m_run == -INFINITY;
    const bool bump = !first && mt > m_run + 8.f;
    const float corr = bump ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
    m_run = first || bump ? mt : m_run;
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    float pr[16], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(sc[r] - mref);  // exp2(-inf) = 0 for masked keys
      ps += pr[r];
    }
    ps += __shfl_xor(ps, 32);
    l_run = l_run * corr + ps;
    if (__any(corr != 1.f)) {
#pragma unroll
      for (int bb = 0; bb < NBW; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[bb][r] *= corr;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int bb = 0; bb < NBW; ++bb) o[bb] = __builtin_amdgcn_mfma_f32_32x32x2f32(b.v[t][bb], pr[t], o[bb], 0, 0, 0);
  };

  // two register sets: the next tile's loads are in flight while a tile is
  // multiplied (every wave runs the same tiles, so the barriers match)
  Tile ta, tb;
  load(ta, 0);
  for (int it = 0; it < ntile; it += 2) {
    if (it + 1 < ntile) load(tb, it + 1);
    compute(ta, it);
    if (it + 1 >= ntile) break;
    if (it + 2 < ntile) load(ta, it + 2);
    compute(tb, it + 1);
  }

  if (q_ok) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* orow = a.out + (size_t)tq * a.nq * HD + (size_t)h * HD + wave * D;
    // register r holds MFMA row i = 8(r/4) + 4 lk + r%4 of every block: dims NBW i .. NBW i + NBW - 1
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      vnb v;
#pragma unroll
      for (int bb = 0; bb < NBW; ++bb) v[bb] = o[bb][r] * inv;
      *reinterpret_cast<vnb*>(orow + NBW * (8 * (r >> 2) + 4 * lk + (r & 3))) = v;
    }
  }
}

}  // namespace qd
