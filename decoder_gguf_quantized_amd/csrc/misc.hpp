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
};

QD_DEV float weight_at(const WView& w, size_t row, int k) {
  const int kp = w.nblk * 32;
  if (w.type == kQ8_0) {
    float d = load_half(w.d + row * w.nblk + (k >> 5));
    return d * (float)reinterpret_cast<const int8_t*>(w.qs)[row * kp + k];
  }
  if (w.type == kQ4_0) {
    const int b = k >> 5, j = k & 31;
    uint32_t byte = w.qs[(row * w.nblk + b) * 16 + (j & 15)];
    uint32_t n = j < 16 ? (byte & 15u) : (byte >> 4);
    float d = load_half(w.d + row * w.nblk + b);
    return d * (float)((int)n - 8);
  }
  return reinterpret_cast<const float*>(w.qs)[row * kp + k];
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

__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int t = blockIdx.x;
  int tok = a.tokens[t];
  if (tok < 0 || tok >= a.vocab) {
    if (threadIdx.x == 0 && a.err) *a.err = 1;
    tok = tok < 0 ? 0 : a.vocab - 1;
  }
  // eight elements per thread per batch: their loads are all issued before the
  // first store, so a row costs one memory round trip per 2048 elements
  for (int k0 = threadIdx.x; k0 < a.hidden; k0 += 256 * 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + 256 * i;
      v[i] = k < a.hidden ? weight_at(a.w, (size_t)tok, k) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + 256 * i;
      if (k < a.hidden) a.out[(size_t)t * a.ldo + k] = v[i];
    }
  }
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
};

__global__ __launch_bounds__(256) void rope_kv_kernel(RopeArgs a) {
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seq = a.dpos ? t : a.seq0;
  const int pos = a.dpos ? a.dpos[t] : a.pos0 + t;
  const int half = a.hd / 2;
  const int nheads = a.nq + 2 * a.nkv;
  const float2* rt = a.rope + (size_t)pos * half;
  for (int hh = wave; hh < nheads; hh += 4) {
    const float* src = a.qkv + (size_t)t * a.ldqkv + (size_t)hh * a.hd;
    const bool is_q = hh < a.nq, is_k = !is_q && hh < a.nq + a.nkv;
    float x1[2], x2[2];
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int i = lane + 64 * r;
      x1[r] = i < half ? src[i] : 0.f;
      x2[r] = i < half ? src[i + half] : 0.f;
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
      dst = base + (((size_t)seq * a.nkv + g) * a.ctx + pos) * a.hd;
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
  int n;
  uint64_t seed;
  uint64_t step;
  float* logits;   // caller's logits buffer for this step
  int* tok_out;    // caller's token buffer for this step
};

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

QD_DEV void argmax_pair_wave(float& v, int& i) {
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (ranks_before(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
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
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int v0 = c * kSampleChunk + 4 * (tid + 256 * k);
    if (v0 >= a.vocab) break;
    u64x4 r;
    if (sampled) {
      u64x4 ctr = {{(uint64_t)(v0 >> 2), a.step, (uint64_t)row, 0ull}};
      r = philox4x64_10(ctr, a.seed, 0ull);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = v0 + w;
      if (v >= a.vocab) break;
      float s = lg[v];
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
};

// Per-step values of a decode step that the replayed graph reads from device
// memory: parameters, positions, input tokens (range-checked), and each
// sequence's RoPE rows at its new position (so decode attention can request
// them without first waiting for the position).
__global__ __launch_bounds__(256) void step_begin_kernel(StepArgs a) {
  const int i = threadIdx.x;
  if (i == 0) *a.d_params = a.params;
  if (i < a.n) {
    a.d_pos[i] = a.pos[i];
    int t = a.dev_tok ? a.dev_tok[i] : a.host_tok[i];
    if (t < 0 || t >= a.vocab) {
      if (a.err) *a.err = 1;
      t = t < 0 ? 0 : a.vocab - 1;
    }
    a.d_tok[i] = t;
  }
  const int per = a.n * a.half;
  for (int e = i; e < 2 * per; e += blockDim.x) {
    const int tbl = e / per, r = e % per, sq = r / a.half, k = r % a.half;
    const float2* src = tbl ? a.rope_l : a.rope_g;
    a.rope_cur[((size_t)tbl * a.max_seqs + sq) * a.half + k] = src[(size_t)a.pos[sq] * a.half + k];
  }
}

}  // namespace qd
