// Small kernels of the forward pass: embedding gather, RMSNorm rows, per-head
// QK-norm + RoPE + KV append, token choice (greedy / Gumbel-max), tensor
// decode for tests, and the per-step parameter upload.
#pragma once
#include "common.hpp"

namespace qd {

// Decoded weight element (row, k) of a repacked tensor.  d * q is exact in f32,
// so this matches any other exact decode bit for bit.
struct WView {
  const uint8_t* qs;
  const uint16_t* d;
  int type;
  int nblk;
  const uint32_t* sd;  // K-quant super-block scales
};

template <int QT>
QD_DEV float weight_at_t(const WView& w, size_t row, int k) {
  const int kp = w.nblk * 32;
  if constexpr (QT == kQ8_0) {
    float d = load_half(w.d + row * w.nblk + (k >> 5));
    return d * (float)reinterpret_cast<const int8_t*>(w.qs)[row * kp + k];
  } else if constexpr (QT == kQ4_0 || QT == kQ4_K) {
    const int b = k >> 5, j = k & 31;
    uint32_t byte = w.qs[(row * w.nblk + b) * 16 + (j & 15)];
    uint32_t n = j < 16 ? (byte & 15u) : (byte >> 4);
    if constexpr (QT == kQ4_K) {  // scale * n - min, rounded once
      const uint32_t sm = w.d[row * w.nblk + b], sd = w.sd[row * (w.nblk >> 3) + (b >> 3)];
      return fmaf(q4k_scale(sm, sd), (float)n, -q4k_min(sm, sd));
    } else {
      float d = load_half(w.d + row * w.nblk + b);
      return d * (float)((int)n - 8);
    }
  } else if constexpr (QT == kQ6_K) {
    const uint32_t sc = (uint32_t)(int32_t)reinterpret_cast<const int8_t*>(w.d)[row * 2 * w.nblk + (k >> 4)];
    const float s = q6k_scale(sc, w.sd[row * (w.nblk >> 3) + (k >> 8)]);
    return s * (float)reinterpret_cast<const int8_t*>(w.qs)[row * kp + k];
  } else {
    return reinterpret_cast<const float*>(w.qs)[row * kp + k];
  }
}

QD_DEV float weight_at(const WView& w, size_t row, int k) {
  switch (w.type) {
    case kQ8_0: return weight_at_t<kQ8_0>(w, row, k);
    case kQ4_0: return weight_at_t<kQ4_0>(w, row, k);
    case kQ4_K: return weight_at_t<kQ4_K>(w, row, k);
    case kQ6_K: return weight_at_t<kQ6_K>(w, row, k);
    default: return weight_at_t<kF32>(w, row, k);
  }
}

// ------------------------------------------------------------ embedding
// Qwen3 walkthrough, Step 2: x = E[token] (a row lookup).  Ids outside
// [0, vocab) are clamped and latch *err.
struct EmbedArgs {
  WView w;
  int hidden, vocab, n;
  const int* tokens;
  float* out;
  int ldo;
  int* err;
};

// One workgroup per token, for the table's weight type QT (a type known at
// compile time keeps the decode free of branches, so all loads of a batch go
// out together).
template <int QT>
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int t = blockIdx.x;
  int tok = a.tokens[t];
  const bool bad = tok < 0 || tok >= a.vocab;
  tok = tok < 0 ? 0 : (tok >= a.vocab ? a.vocab - 1 : tok);
  // sixteen elements per thread per batch: their loads are all issued before
  // the first store (loads and stores share one in-order counter, so a load
  // behind a store waits for it), so a row of up to 4,096 elements costs one
  // memory round trip; indices past the row read its last element
  for (int k0 = threadIdx.x; k0 < a.hidden; k0 += 256 * 16) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = weight_at_t<QT>(a.w, (size_t)tok, min(k0 + 256 * i, a.hidden - 1));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = k0 + 256 * i;
      if (k < a.hidden) a.out[(size_t)t * a.ldo + k] = v[i];
    }
  }
  if (bad && threadIdx.x == 0 && a.err) *a.err = 1;  // after the loads: ids outside [0, vocab) latch the error
}

// ------------------------------------------------------------ RMSNorm rows
// Qwen3 walkthrough, Step 3: y = x * rsqrt(mean(x^2) + eps) * w.  With add = 1
// the result is added into out (sandwich norms: x += RMSNorm(y)).
struct NormArgs {
  const float* x;
  int ldx;
  const float* w;
  float eps;
  int n;
  float* out;
  int ldo;
  int add;
};

__global__ __launch_bounds__(256) void rmsnorm_kernel(NormArgs a) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* xr = a.x + (size_t)t * a.ldx;
  float ss = 0.f;
  for (int k = tid; k < a.n; k += 256) ss += xr[k] * xr[k];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float scale = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)a.n + a.eps);
  float* orow = a.out + (size_t)t * a.ldo;
  for (int k = tid; k < a.n; k += 256) {
    float v = xr[k] * scale * a.w[k];
    if (a.add) orow[k] += v; else orow[k] = v;
  }
}

// ------------------------------------------------------------ QK-norm + RoPE + KV append
// Qwen3 walkthrough, Steps 4-5: per-head RMSNorm of q and k (Qwen3), then the
// half-split rotation of pairs (d, d + hd/2) by angle = f32(pos) * inv_freq[d]
// (a single f32 product), then k and v are appended to the cache.  Synsema's
// qwen3 file orders the norm before the rotation.  cos/sin come from a table
// built at load time: the double-precision cos/sin of that f32 angle, rounded
// once to f32 (angles reach thousands of radians).
struct RopeArgs {
  const float* qkv;     // [n][(nq + 2 nkv) hd]
  int ldqkv;
  float* q_out;         // [n][nq hd]
  float* kc;            // layer base of the cache: [B][nkv][ctx][hd]
  float* vc;
  int ctx, nq, nkv, hd;
  const float* q_norm;  // [hd] or null
  const float* k_norm;
  float eps;
  const float2* rope;   // [ctx][hd/2] (cos, sin) of f32(pos) * inv_freq[i]
  int seq0, pos0;       // prefill: token t -> (seq0, pos0 + t)
  const int* dpos;      // decode (non-null): token t -> (seq t, dpos[t])
  const float* bias;    // [(nq + 2 nkv) hd] q|k|v projection bias added first, or null
  KvMap map;            // cache layout
};

// Grid (token, group of four heads): one wave per head, so every wave makes a
// single round of loads (a wave looping over heads waited on each head's loads
// in turn).  No barriers: a wave past the last head returns.
__global__ __launch_bounds__(256) void rope_kv_kernel(RopeArgs a) {
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seq = a.dpos ? t : a.seq0;
  const int pos = a.dpos ? a.dpos[t] : a.pos0 + t;
  const int half = a.hd / 2;
  const int nheads = a.nq + 2 * a.nkv;
  const float2* rt = a.rope + (size_t)pos * half;
  const int hh = (int)blockIdx.y * 4 + wave;
  if (hh < nheads) {
    const float* src = a.qkv + (size_t)t * a.ldqkv + (size_t)hh * a.hd;
    const bool is_q = hh < a.nq, is_k = !is_q && hh < a.nq + a.nkv;
    float x1[2], x2[2];
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int i = lane + 64 * r;
      x1[r] = i < half ? src[i] : 0.f;
      x2[r] = i < half ? src[i + half] : 0.f;
      if (a.bias && i < half) {
        x1[r] += a.bias[(size_t)hh * a.hd + i];
        x2[r] += a.bias[(size_t)hh * a.hd + i + half];
      }
      ss += x1[r] * x1[r] + x2[r] * x2[r];
    }
    const float* nw = is_q ? a.q_norm : (is_k ? a.k_norm : nullptr);
    if (nw) {
      ss = wave_sum(ss);
      const float scale = 1.0f / sqrtf(ss / (float)a.hd + a.eps);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        int i = lane + 64 * r;
        if (i < half) {
          x1[r] = x1[r] * scale * nw[i];
          x2[r] = x2[r] * scale * nw[i + half];
        }
      }
    }
    float* dst;
    if (is_q) {
      dst = a.q_out + (size_t)t * a.nq * a.hd + (size_t)hh * a.hd;
    } else {
      const int g = is_k ? hh - a.nq : hh - a.nq - a.nkv;
      float* base = is_k ? a.kc : a.vc;
      dst = base + kv_row(a.map, a.nkv, a.ctx, seq, g, pos) * a.hd;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int i = lane + 64 * r;
      if (i >= half) continue;
      float y1 = x1[r], y2 = x2[r];
      if (is_q || is_k) {
        const float2 cs = rt[i];
        y1 = x1[r] * cs.x - x2[r] * cs.y;
        y2 = x1[r] * cs.y + x2[r] * cs.x;
      }
      dst[i] = y1;
      dst[i + half] = y2;
    }
  }
}

// ------------------------------------------------------------ token choice
// Qwen3 walkthrough, Step 8: temperature 0 -> argmax; otherwise a draw from
// softmax(logits / T), taken here as argmax(logits / T + Gumbel) with the
// uniforms from Philox4x64-10, counter (v / 4, step, row, 0), key (seed, 0),
// word v % 4.  Stage 1: one workgroup per (4096-entry vocab chunk, row).
constexpr int kSampleChunk = 4096;

// Per-step values that a replayed decode graph reads from device memory.
struct StepParams {
  float temperature;
  float top_p;
  int n;
  uint64_t seed;
  uint64_t step;
  float* logits;   // caller's logits buffer for this step
  int* tok_out;    // caller's token buffer for this step
};

// ------------------------------------------------------------ top-p cut
// Walkthrough, Step 8 sampler: with probabilities p = softmax(logits / T) in
// descending order (equal ones by lower index), keep the first
// count(running sum < top_p) + 1 tokens.  For T > 0 the probability order is
// the logit order, so tokens are ranked by an order-preserving key of the
// logit.  The running sums use fixed-point weights W = floor(2^40 * e) of
// e = 2^((l - lmax) * log2(e) / T) (f32), summed as 64-bit integers: exact and
// independent of summation order.  A token is kept when the weight of the
// tokens ranked before it is below top_p * Z (Z = sum of all weights), which is
// count(running sum < top_p) + 1 of the page.  The boundary token's key is
// found by radix selection over the key's four bytes (one pass over the row
// each), and where the boundary falls inside a run of equal logits, the index
// of the last kept one by one more pass.  Result per row: tokens with key >
// cut_key, or key == cut_key and index <= cut_idx, are kept.  top_p >= 1,
// T = 0 or a non-finite logit keep every token (cut_key = 0).

// Key that orders floats like their values (-0 and +0 alike; NaN excluded by
// the caller).
QD_DEV uint32_t order_key(float l) {
  const uint32_t b = __float_as_uint(l == 0.f ? 0.f : l);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

QD_DEV float key_value(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// floor(2^40 * e) for e in [0, 1], exact (e = m * 2^(E - 23)); a row's sum stays
// below 2^59.
QD_DEV uint64_t fixed40(float e) {
  const uint32_t b = __float_as_uint(e);
  if (b < 0x00800000u) return 0ull;  // zero or below 2^-126
  const int E = (int)(b >> 23) - 127;
  const uint64_t m = (b & 0x7FFFFFu) | 0x800000u;
  const int sh = E + 17;
  return sh >= 0 ? (m << sh) : (sh > -64 ? (m >> -sh) : 0ull);
}

QD_DEV uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += (uint64_t)__shfl_xor((long long)v, o);
  return v;
}

// The cut is found in passes over the row, each a launch of topp_pass_kernel
// with grid (kTopPChunks, rows): workgroup c takes the c-th chunk of the row.
// pass 0: each chunk's max (and whether it holds a non-finite logit);
// pass 1: the coarse histogram; passes 2..5: select in the previous level's
// histogram, then histogram the next byte of the key among the candidates;
// pass 6 (one workgroup per row): select the last byte, then resolve ties.
// Histograms are sums of 64-bit integer weights with atomic adds, so every
// order of the adds gives the same sums; every workgroup of a pass repeats the
// selection from the same histogram and state and reaches the same result, so
// the workgroups of a pass never wait for one another.  Buffers: the level-c
// histogram (c = 0 coarse, 1..4 key bytes) is accumulated in hist[c % 3] by
// pass c + 1, which also clears hist[(c + 1) % 3] (read last by the pass
// before); the state is written by each pass's first chunk into state[pass % 2]
// and read by the next pass from state[(pass - 1) % 2].
constexpr int kTopPChunks = 64;

struct TopPState {
  float lmax;
  int mode;                       // 0: cut in progress, 1: decided (keep all)
  double target;                  // top_p * Z
  unsigned long long above;       // weight of the tokens ranked before the candidates
  unsigned long long tie_mass;    // weight of the selected bin
  uint32_t prefix, mask;          // key bytes selected so far
  int cb;                         // coarse bin of the candidates
};

struct TopPArgs {
  const float* logits;
  int ld, vocab, rows;
  float temperature, top_p;
  uint32_t* cut_key;  // [rows]
  int* cut_idx;       // [rows]
  const StepParams* sp;  // if non-null: logits, temperature, top_p come from here
  float* pmax;        // [rows][kTopPChunks]
  int* pbad;          // [rows][kTopPChunks]
  unsigned long long* hist;  // [3][rows][256]
  TopPState* state;   // [2][rows]
  int pass;
};

// Device buffers of the passes for up to `rows` rows.
struct TopPScratch {
  float* pmax;                // [rows][kTopPChunks]
  int* pbad;                  // [rows][kTopPChunks]
  unsigned long long* hist;   // [3][rows][256]
  TopPState* state;           // [2][rows]
};

__global__ __launch_bounds__(256) void topp_pass_kernel(TopPArgs a) {
  constexpr int NW = 4;
  __shared__ unsigned long long h[NW][256];  // per-wave histograms; h[0] also holds a read level
  __shared__ float sm_max[NW];
  __shared__ int sm_bad[NW];
  __shared__ unsigned long long sm_sel[2];
  __shared__ int sm_i[2];
  __shared__ int sm_cnt[NW];
  if (a.sp) {
    a.logits = a.sp->logits;
    a.temperature = a.sp->temperature;
    a.top_p = a.sp->top_p;
  }
  const int chunk = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* lg = a.logits + (size_t)row * a.ld;
  const int V = a.vocab;
  const int per = (V + kTopPChunks - 1) / kTopPChunks;
  const int c0 = min(V, chunk * per), c1 = min(V, c0 + per);
  unsigned long long* hrow = a.hist + (size_t)row * 256;
  const size_t hstride = (size_t)a.rows * 256;
  auto hbuf = [&](int c) { return hrow + (size_t)(c % 3) * hstride; };
  TopPState* out_state = a.state + (size_t)(a.pass % 2) * a.rows + row;
  const TopPState* in_state = a.state + (size_t)((a.pass + 1) % 2) * a.rows + row;
  auto keep_all = [&]() {  // the first chunk records the result and the decision
    if (chunk == 0 && tid == 0) {
      a.cut_key[row] = 0u;
      a.cut_idx[row] = 0x7fffffff;
      TopPState st{};
      st.mode = 1;
      *out_state = st;
    }
  };
  if (!(a.temperature > 0.f) || !(a.top_p < 1.f)) {
    keep_all();
    return;
  }
  if (a.pass == 0) {  // chunk max; a non-finite logit keeps every token
    float mx = -INFINITY;
    int bad = 0;
    for (int v = c0 + tid; v < c1; v += 256) {
      const float l = lg[v];
      bad |= !isfinite(l);
      mx = fmaxf(mx, l);
    }
    mx = wave_max(mx);
    bad = __ballot(bad) != 0ull;
    if (lane == 0) {
      sm_max[wave] = mx;
      sm_bad[wave] = bad;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NW; ++w) {
        mx = fmaxf(mx, sm_max[w]);
        bad |= sm_bad[w];
      }
      a.pmax[(size_t)row * kTopPChunks + chunk] = fmaxf(sm_max[0], mx);
      a.pbad[(size_t)row * kTopPChunks + chunk] = bad | sm_bad[0];
    }
    if (chunk == 0) hbuf(0)[tid] = 0ull;  // accumulated by pass 1
    return;
  }
  TopPState st;
  if (a.pass == 1) {
    st = TopPState{};
    float lmax = -INFINITY;
    int anybad = 0;
    for (int c = 0; c < kTopPChunks; ++c) {
      lmax = fmaxf(lmax, a.pmax[(size_t)row * kTopPChunks + c]);
      anybad |= a.pbad[(size_t)row * kTopPChunks + c];
    }
    if (anybad) {
      keep_all();
      return;
    }
    st.lmax = lmax;
  } else {
    st = *in_state;
    if (st.mode) {
      if (chunk == 0 && tid == 0) *out_state = st;
      return;
    }
  }
  const float cw = 1.4426950408889634f / a.temperature;
  auto weight = [&](float l) { return fixed40(exp2f((l - st.lmax) * cw)); };
  // coarse bin of a logit by its distance from the max, 1/8 of a log2 unit of
  // weight per bin (the last bin takes the rest).  Monotone in the logit, so a
  // bin is a contiguous range of keys; it spreads a row over many bins, which
  // the key's top byte does not (logits of one row share a few exponents).
  auto cbin = [&](float l) { return (int)fminf((st.lmax - l) * cw * 8.0f, 255.0f); };
  // selection over the 256 bins of h[0] (bin order given by `desc`: key bytes
  // run high to low from bin 255, coarse bins from bin 0): the bin where the
  // running weight crosses the target, the weight before it and its own weight
  auto select = [&](bool desc, unsigned long long base, int& sel, unsigned long long& before,
                    unsigned long long& mass) {
    if (wave == 0) {
      unsigned long long b4[4], loc = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b4[j] = h[0][desc ? 255 - 4 * lane - j : 4 * lane + j];
        loc += b4[j];
      }
      unsigned long long inc = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long t = (unsigned long long)__shfl_up((long long)inc, o);
        if (lane >= o) inc += t;
      }
      unsigned long long run = base + (inc - loc);
      int found = -1;
      unsigned long long f_before = 0ull, f_bin = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (found < 0 && b4[j] > 0ull && (double)run < st.target && (double)(run + b4[j]) >= st.target) {
          found = desc ? 255 - 4 * lane - j : 4 * lane + j;
          f_before = run;
          f_bin = b4[j];
        }
        run += b4[j];
      }
      if (lane == 0) sm_i[0] = -1;
      if (found >= 0) {  // one lane at most: the running sums increase
        sm_i[0] = found;
        sm_sel[0] = f_before;
        sm_sel[1] = f_bin;
      }
    }
    __syncthreads();
    sel = sm_i[0];
    before = sm_sel[0];
    mass = sm_sel[1];
    __syncthreads();  // everyone has read the selection before h is cleared again
  };
  // the previous level's histogram into h[0]; after the coarse level, its total is Z
  if (a.pass >= 2) {
    h[0][tid] = hbuf(a.pass - 2)[tid];
    __syncthreads();
    if (a.pass == 2) {
      if (tid < 64) {
        unsigned long long z = h[0][tid] + h[0][tid + 64] + h[0][tid + 128] + h[0][tid + 192];
        z = wave_sum_u64(z);
        if (tid == 0) sm_sel[0] = z;
      }
      __syncthreads();
      const unsigned long long Z = sm_sel[0];
      __syncthreads();
      st.target = (double)a.top_p * (double)Z;  // Z < 2^59: rounded to double, relative 2^-53
      if (st.target < 0.5) st.target = 0.5;     // top_p <= 0: the first token only
      if (st.target > (double)Z) {
        keep_all();
        return;
      }
      int cb;
      unsigned long long above, tie_mass;
      select(false, 0ull, cb, above, tie_mass);
      if (cb < 0) {
        keep_all();
        return;
      }
      st.cb = cb;
      st.above = above;
      st.tie_mass = tie_mass;
    } else {  // key byte level pass - 3
      int d;
      unsigned long long before, mass;
      select(true, st.above, d, before, mass);
      if (d < 0) {  // guard: the candidates' weight cannot reach the target
        keep_all();
        return;
      }
      const int sh = 24 - 8 * (a.pass - 3);
      st.above = before;
      st.tie_mass = mass;
      st.prefix |= (uint32_t)d << sh;
      st.mask |= 255u << sh;
    }
  }
  if (a.pass <= 5) {
    // this chunk's share of the next level: the coarse bins (pass 1) or key
    // byte pass - 2 among the candidates (coarse bin cb, key bytes so far)
    for (int i = tid; i < NW * 256; i += 256) (&h[0][0])[i] = 0ull;
    __syncthreads();
    if (a.pass == 1) {
      for (int v = c0 + tid; v < c1; v += 256) {
        const float l = lg[v];
        atomicAdd(&h[wave][cbin(l)], weight(l));
      }
    } else {
      const int sh = 24 - 8 * (a.pass - 2);
      for (int v = c0 + tid; v < c1; v += 256) {
        const float l = lg[v];
        const uint32_t k = order_key(l);
        if ((k & st.mask) == st.prefix && cbin(l) == st.cb) atomicAdd(&h[wave][(k >> sh) & 255u], weight(l));
      }
    }
    __syncthreads();
    unsigned long long t = 0ull;
    for (int w = 0; w < NW; ++w) t += h[w][tid];
    if (t) atomicAdd(hbuf(a.pass - 1) + tid, t);
    if (chunk == 0) {
      hbuf(a.pass)[tid] = 0ull;  // accumulated by the next pass
      if (tid == 0) *out_state = st;
    }
    return;
  }
  // pass 6: prefix = key of the boundary token, above = weight of the larger
  // keys, tie_mass = weight of the tokens with the boundary key (equal weights)
  int cut = 0x7fffffff;
  const unsigned long long w1 = weight(key_value(st.prefix));
  const unsigned long long cnt = w1 ? st.tie_mass / w1 : 0ull;
  const double need = w1 ? ceil((st.target - (double)st.above) / (double)w1) : 0.0;  // ties to keep, >= 1
  if (w1 && need < (double)cnt) {
    const int n_need = (int)need;
    // the n_need-th token (in index order) with the boundary key
    const int seg = (V + 255) / 256, b0 = min(V, tid * seg), b1 = min(V, b0 + seg);
    int c_t = 0;
    for (int v = b0; v < b1; ++v) c_t += order_key(lg[v]) == st.prefix;
    int inc = c_t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    if (lane == 63) sm_cnt[wave] = inc;
    if (tid == 0) sm_i[1] = 0x7fffffff;
    __syncthreads();
    int before = inc - c_t;
    for (int w = 0; w < wave; ++w) before += sm_cnt[w];
    if (before < n_need && before + c_t >= n_need) {
      int r = before;
      for (int v = b0; v < b1; ++v)
        if (order_key(lg[v]) == st.prefix && ++r == n_need) {
          sm_i[1] = v;
          break;
        }
    }
    __syncthreads();
    cut = sm_i[1];
  }
  if (tid == 0) {
    a.cut_key[row] = st.prefix;
    a.cut_idx[row] = cut;
  }
}

struct SampleArgs {
  const float* logits;
  int ld, vocab, rows;
  float temperature;
  uint64_t seed, step;
  float* part_v;   // [rows][nchunk]
  int* part_i;
  int nchunk;
  int* out;        // [rows]
  int* out2;       // optional second copy
  const StepParams* sp;  // if non-null: logits, out, temperature, seed, step come from here
  const uint32_t* cut_key;  // if non-null: top-p cut per row (see topp_pass_kernel)
  const int* cut_idx;
  const int* seq;  // if non-null: sequence slot of each row, the row index of the random stream
};

QD_DEV void sample_resolve(SampleArgs& a) {
  if (a.sp) {
    a.logits = a.sp->logits;
    a.out = a.sp->tok_out;
    a.temperature = a.sp->temperature;
    a.seed = a.sp->seed;
    a.step = a.sp->step;
  }
}

__global__ __launch_bounds__(256) void sample_stage1_kernel(SampleArgs a) {
  sample_resolve(a);
  __shared__ float sv[4];
  __shared__ int si[4];
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const float* lg = a.logits + (size_t)row * a.ld;
  float best = 0.f;
  int bi = 0x7fffffff;
  bool have = false;
  const bool sampled = a.temperature > 0.f;
  const uint32_t ck = a.cut_key ? a.cut_key[row] : 0u;
  const int ci = a.cut_key ? a.cut_idx[row] : 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int v0 = c * kSampleChunk + 4 * (tid + 256 * k);
    if (v0 >= a.vocab) break;
    u64x4 r;
    if (sampled) {
      u64x4 ctr = {{(uint64_t)(v0 >> 2), a.step, (uint64_t)(a.seq ? a.seq[row] : row), 0ull}};
      r = philox4x64_10(ctr, a.seed, 0ull);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = v0 + w;
      if (v >= a.vocab) break;
      float s = lg[v];
      if (a.cut_key) {  // tokens outside the top-p nucleus take no part
        const uint32_t k = order_key(s);
        if (k < ck || (k == ck && v > ci)) continue;
      }
      if (sampled) {
        float u = philox_uniform(r.v[w]);
        s = s / a.temperature - logf(-logf(u));
      }
      if (!have || ranks_before(s, v, best, bi)) {
        best = s;
        bi = v;
        have = true;
      }
    }
  }
  if (!have) {
    best = -INFINITY;
    bi = 0x7fffffff;
  }
  argmax_pair_wave(best, bi);
  if ((tid & 63) == 0) {
    sv[tid >> 6] = best;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (ranks_before(sv[w], si[w], best, bi)) {
        best = sv[w];
        bi = si[w];
      }
    a.part_v[(size_t)row * a.nchunk + c] = best;
    a.part_i[(size_t)row * a.nchunk + c] = bi;
  }
}

__global__ __launch_bounds__(64) void sample_stage2_kernel(SampleArgs a) {
  sample_resolve(a);
  const int row = blockIdx.x, lane = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  bool have = false;
  for (int c = lane; c < a.nchunk; c += 64) {
    float v = a.part_v[(size_t)row * a.nchunk + c];
    int i = a.part_i[(size_t)row * a.nchunk + c];
    if (!have || ranks_before(v, i, best, bi)) {
      best = v;
      bi = i;
      have = true;
    }
  }
  argmax_pair_wave(best, bi);
  if (lane == 0) {
    a.out[row] = bi;
    if (a.out2) a.out2[row] = bi;
  }
}

// The greedy token of one row from the LM head GEMV's per-wave choices
// (part_v / part_i [nchunk]): each thread takes eight entries per round with
// all loads in flight at once (a single wave looping over thousands of
// entries would pay one memory round trip per 64), then a wave and a
// workgroup reduction in the sampler's ranking.
__global__ __launch_bounds__(1024) void argmax_waves_kernel(SampleArgs a) {
  sample_resolve(a);
  constexpr int kPer = 8;
  __shared__ float sv[16];
  __shared__ int si[16];
  const int tid = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int c0 = 0; c0 < a.nchunk; c0 += 1024 * kPer) {
    float v[kPer];
    int id[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int c = c0 + tid + 1024 * k;
      const bool ok = c < a.nchunk;
      v[k] = ok ? a.part_v[c] : -INFINITY;
      id[k] = ok ? a.part_i[c] : 0x7fffffff;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (ranks_before(v[k], id[k], best, bi)) {
        best = v[k];
        bi = id[k];
      }
  }
  argmax_pair_wave(best, bi);
  if ((tid & 63) == 0) {
    sv[tid >> 6] = best;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid < 64) {
    best = tid < 16 ? sv[tid] : -INFINITY;
    bi = tid < 16 ? si[tid] : 0x7fffffff;
    argmax_pair_wave(best, bi);
    if (tid == 0) {
      a.out[0] = bi;
      if (a.out2) a.out2[0] = bi;
    }
  }
}

// ------------------------------------------------------------ tests: decode a tensor
struct DequantArgs {
  WView w;
  const int* row_map;   // device row of logical row r, or null (identity + row_off)
  int row_off, rows, cols;
  int pair;             // 1 = gate rows of the gate/up interleave, 2 = up rows
  float* out;
};

__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const int r = blockIdx.x;
  size_t dr;
  if (a.pair) dr = (size_t)((r >> 5) * 64 + (r & 31) + (a.pair == 2 ? 32 : 0));
  else dr = (size_t)(r + a.row_off);
  for (int k = threadIdx.x; k < a.cols; k += 256) a.out[(size_t)r * a.cols + k] = weight_at(a.w, dr, k);
}

// ------------------------------------------------------------ per-step parameters
// Copies the step's input tokens and positions into library buffers, so the
// rest of the step reads them from fixed device addresses.
struct StepArgs {
  int n;
  int pos[64];
  int host_tok[64];
  int seq[64];          // sequence slot of each row (written to d_seq if non-null)
  int* d_seq;
  int tbl_n;            // page-table entries to set before the step (paged cache)
  int tbl_idx[64], tbl_val[64];
  int* d_table;
  const int* dev_tok;   // non-null: tokens come from device memory
  int vocab;
  int* d_pos;
  int* d_tok;
  int* err;
  StepParams params;
  StepParams* d_params;
  const float2* rope_g;  // RoPE tables [ctx][half] (full-attention and sliding-window layers)
  const float2* rope_l;
  float2* rope_cur;      // [2][max_seqs][half]: each sequence's rows at its new position
  int half, max_seqs;
  float* acc_clear;      // decode attention's layer-0 accumulators to zero (models with an odd
  long acc_n;            // number of layers, where the last layer does not clear them), or null
};

// Per-step values of a decode step that the replayed graph reads from device
// memory: parameters, positions, input tokens (range-checked), and each
// sequence's RoPE rows at its new position (so decode attention can request
// them without first waiting for the position).
__global__ __launch_bounds__(256) void step_begin_kernel(StepArgs a) {
  const int i = threadIdx.x;
  if (i == 0) *a.d_params = a.params;
  if (i < a.tbl_n) a.d_table[a.tbl_idx[i]] = a.tbl_val[i];
  if (i < a.n) {
    if (a.d_seq) a.d_seq[i] = a.seq[i];
    a.d_pos[i] = a.pos[i];
    int t = a.dev_tok ? a.dev_tok[i] : a.host_tok[i];
    if (t < 0 || t >= a.vocab) {
      if (a.err) *a.err = 1;
      t = t < 0 ? 0 : a.vocab - 1;
    }
    a.d_tok[i] = t;
  }
  if (a.acc_clear)
    for (long e = i; e < a.acc_n; e += blockDim.x) a.acc_clear[e] = 0.f;
  const int per = a.n * a.half;
  for (int e = i; e < 2 * per; e += blockDim.x) {
    const int tbl = e / per, r = e % per, sq = r / a.half, k = r % a.half;
    const float2* src = tbl ? a.rope_l : a.rope_g;
    a.rope_cur[((size_t)tbl * a.max_seqs + sq) * a.half + k] = src[(size_t)a.pos[sq] * a.half + k];
  }
}

// ------------------------------------------------------------ paged-cache upkeep
// Page-table entries set in stream order (the host hands out pages and passes
// the new entries by value).
struct TableSet {
  int n;
  int idx[64], val[64];
  int* table;
};

__global__ __launch_bounds__(64) void table_set_kernel(TableSet t) {
  if ((int)threadIdx.x < t.n) t.table[t.idx[threadIdx.x]] = t.val[threadIdx.x];
}

// Copy preset K and V rows ([nkv][n][hd] each) of one (sequence, layer) into
// the cache at positions j0..n-1 (j0 > 0 for a ring that keeps only the last
// positions).  Grid (n - j0, nkv, 2: K / V), hd / 4 threads.
struct KvScatter {
  const float* src_k;
  const float* src_v;
  float* kc;            // layer base of the caches
  float* vc;
  int n, nkv, ctx, hd, seq;
  KvMap map;
  int j0;
};

__global__ __launch_bounds__(64) void kv_scatter_kernel(KvScatter a) {
  const int j = a.j0 + (int)blockIdx.x, g = blockIdx.y, which = blockIdx.z, e = threadIdx.x;
  const float4* src = reinterpret_cast<const float4*>((which ? a.src_v : a.src_k) + ((size_t)g * a.n + j) * a.hd);
  float4* dst = reinterpret_cast<float4*>((which ? a.vc : a.kc) + kv_row(a.map, a.nkv, a.ctx, a.seq, g, j) * a.hd);
  if (e < a.hd / 4) dst[e] = src[e];
}

}  // namespace qd
