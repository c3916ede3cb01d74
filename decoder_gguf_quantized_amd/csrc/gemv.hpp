// Decode projection: y[m][n] = sum_k W[n][k] * x[m][k] for a handful of input
// rows (decode batch, 1..16), W block-quantized in HBM.
//
// Qwen3 walkthrough, Step 5 (Q/K/V/O projections `x @ W.T`) and Step 6 (SwiGLU);
// Synsema "Choose the engine": the weights stay quantized and are multiplied in
// f32 -- each block is decoded in registers (int8 / nibble -> f32, fp16 scale
// applied once per block) and every product and sum is f32.
//
// Bandwidth design (decode is a weight stream, ~1 byte per weight):
//   * scales and quants are split (SoA) so a lane issues one 16-byte load per
//     unit (Q8_0: 16 weights, Q4_0: a whole 32-weight block, F32: 4 weights);
//     64 lanes read 1 KB contiguous per row: fully coalesced.
//   * each wave streams R rows at once with U units per lane in flight per row
//     (R*U 16-byte loads per lane before the first use); the input rows sit in
//     LDS (RMSNorm prologue fused), so a unit's activations are read once for
//     all R rows.  The first row group's weights are requested before the
//     prologue, so the input staging overlaps the first weight fetch.
//   * the reduction over the 64 lanes is a DPP tree; a wave keeps its finished
//     outputs in a register (one lane each) and writes them all at the end with
//     the mode's epilogue (store, residual add, or gate/up pair with the
//     activation: act(gate) * up).  The ring of weight tiles then issues only
//     loads, the same number on every path, so each wait is for exactly the
//     tile about to be used (loads and stores share one in-order counter: a
//     store, or a conditional load, inside the ring turns every later wait into
//     a wait for all loads in flight).
//   * Q8_0: int8 -> f32 is one SDWA conversion per weight.  Q4_0: nibbles are
//     masked a word at a time into fp16 subnormals that the mixed-precision FMA
//     reads directly (dot32_q4_raw4); the offset 8 is folded into the block as
//     -8 * sum(x over the block), so the per-weight cost is one FMA and 5/8 of
//     a mask or shift.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace qd {

enum { kModeStore = 0, kModeAdd = 1, kModePairSilu = 2, kModePairGelu = 3 };

struct GemvArgs {
  const uint8_t* qs;     // Q8_0: int8 [rows][kp]; Q4_0: u8 [rows][nblk][16]; F32: f32 [rows][kp]
  const uint16_t* d;     // fp16 scales [rows][nblk] (quantized types)
  int rows;              // weight rows
  int nblk;              // 32-value blocks per row, kp = 32 * nblk
  const float* x;        // input rows [m][ldx]; columns [0, kp) are read
  int ldx;
  const float* norm_w;   // RMSNorm gain [kp], or null for no prologue norm
  float eps;
  float* y;              // output rows [m][ldy]
  int ldy;
  int m;                 // input rows in this launch (<= template M)
  float* const* y_ind;   // if non-null, the output base is *y_ind + y_off (graph replays)
  long y_off;
  // Residual prologue (sandwich norms): if res_add is non-null, the input row
  // is h = x + RMSNorm(res_add) * res_w (rows [m][ldx]), which the norm_w
  // prologue then normalises; workgroup 0 writes h to res_out (if non-null).
  const float* res_add;
  const float* res_w;
  float* res_out;
  const float* bias;     // store mode: y[n] += bias[n] (qwen2's q/k/v bias adds), or null
  const uint32_t* sd;    // K-quants: super-block scales [rows][nblk / 8]; `d` then holds the
                         // per-sub-block words (Q4_K u16, Q6_K int8 per 16 values)
  // Input from decode attention's accumulators instead of x: element k of row
  // mi is sum_b xd[b][mi][k] / sum_b xl[b][mi][k / xhd] over the kAccCopies
  // blocks b (xcstride floats apart; rows [m][ldx] and [m][ldx / xhd]): the
  // split softmax's final division.
  const float* xd;
  const float* xl;
  int xhd;
  long xcstride;
  // Greedy token choice fused into the store epilogue (the LM head of one input
  // row): each wave keeps the best (value, lowest index) of the rows it stores,
  // ranked as the sampler ranks them (NaN above every number), and writes it to
  // amax_v / amax_i [nwaves]; a one-wave pass then reduces the waves' results.
  // Null: no argmax.
  float* amax_v;
  int* amax_i;
};

// Input row mi, floats 4 k4 .. 4 k4 + 3, in two steps: the loads (always
// issued, at a clamped in-bounds index, so every thread issues the same loads)
// and the arithmetic on them (zero past the row or past the launch's rows).
// ACC: the row comes from decode attention's accumulators, kAccCopies blocks
// summed and divided by their softmax denominators (a separate instantiation,
// so that the plain kernels keep their register budget).
template <bool ACC>
struct XRaw {
  float4 u[ACC ? kAccCopies : 1];
  float l[ACC ? kAccCopies : 1];
};

template <bool ACC>
QD_DEV XRaw<ACC> load_x4_raw(const GemvArgs& a, int mi, int k4, bool ok) {
  const int m = min(mi, a.m - 1), k = ok ? k4 : 0;
  XRaw<ACC> r;
  if constexpr (ACC) {
#pragma unroll
    for (int b = 0; b < kAccCopies; ++b) {  // every block's loads go out together
      r.u[b] = reinterpret_cast<const float4*>(a.xd + b * a.xcstride + (size_t)m * a.ldx)[k];
      r.l[b] = a.xl[b * a.xcstride + (size_t)m * (a.ldx / a.xhd) + (4 * k) / a.xhd];
    }
  } else {
    r.u[0] = reinterpret_cast<const float4*>(a.x)[(size_t)m * (a.ldx / 4) + k];
  }
  return r;
}

template <bool ACC>
QD_DEV float4 x4_value(const GemvArgs& a, const XRaw<ACC>& r, int mi, bool ok) {
  if (!ok || mi >= a.m) return make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (ACC) {
    float4 o = r.u[0];
    float l = r.l[0];
#pragma unroll
    for (int b = 1; b < kAccCopies; ++b) {
      o.x += r.u[b].x;
      o.y += r.u[b].y;
      o.z += r.u[b].z;
      o.w += r.u[b].w;
      l += r.l[b];
    }
    const float q = 1.0f / l;
    return make_float4(o.x * q, o.y * q, o.z * q, o.w * q);
  }
  return r.u[0];
}

// Activations from the hardware exp2 and reciprocal (about one ulp each): a
// precise division and expf cost ~30 instructions per output, which the
// gate/up GEMV (bound by its vector ALU) pays once per row pair.
//   silu(g)      = g / (1 + e^-g)
//   gelu_tanh(x) = 0.5 x (1 + tanh u) = x / (1 + e^-2u),  u = sqrt(2/pi) (x + 0.044715 x^3)
// Far tails: e^-g overflows to inf and the output is -0 (silu) / -0 (gelu);
// e^-g underflows to 0 and the output is g.
QD_DEV float act_silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}
QD_DEV float act_gelu_tanh(float x) {
  const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);  // sqrt(2/pi) (x + 0.044715 x^3)
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.8853900817779268f * u));
}

// Gate/up interleave used by the pair modes: weight rows [64b, 64b+32) hold gate
// rows [32b, 32b+32) and [64b+32, 64b+64) the matching up rows.
QD_DEV int pair_gate_row(int n) { return (n >> 5) * 64 + (n & 31); }

// Q4_0 / Q8_0 decode from unsigned bytes: with u = q + c (c = 8 for a nibble,
// 128 for an int8 byte with its sign bit flipped), d q = fma(d, u, -c d).  Both
// products are exact in f32 (an fp16 scale times an integer below 2^8), and so
// is their difference, so the fma rounds nothing and the value equals d * q
// (an exact zero comes out +0).  Byte E of w converts in one instruction
// (V_CVT_F32_UBYTE0..3, written out: the compiler would otherwise extract a
// masked nibble with a bit-field instruction first).
template <int E>
QD_DEV float dq_byte(float d, float cd, uint32_t w) {
  float f;
  if constexpr (E == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(w));
  else if constexpr (E == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(w));
  else if constexpr (E == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(w));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(w));
  return fmaf(d, f, cd);
}

QD_DEV float dot16_q8(uint4 w, const float4& a, const float4& b, const float4& c, const float4& e) {
  float s = 0.f;
  s += (float)(int8_t)(w.x) * a.x;
  s += (float)(int8_t)(w.x >> 8) * a.y;
  s += (float)(int8_t)(w.x >> 16) * a.z;
  s += (float)(int8_t)(w.x >> 24) * a.w;
  s += (float)(int8_t)(w.y) * b.x;
  s += (float)(int8_t)(w.y >> 8) * b.y;
  s += (float)(int8_t)(w.y >> 16) * b.z;
  s += (float)(int8_t)(w.y >> 24) * b.w;
  s += (float)(int8_t)(w.z) * c.x;
  s += (float)(int8_t)(w.z >> 8) * c.y;
  s += (float)(int8_t)(w.z >> 16) * c.z;
  s += (float)(int8_t)(w.z >> 24) * c.w;
  s += (float)(int8_t)(w.w) * e.x;
  s += (float)(int8_t)(w.w >> 8) * e.y;
  s += (float)(int8_t)(w.w >> 16) * e.z;
  s += (float)(int8_t)(w.w >> 24) * e.w;
  return s;
}

// Activations per lane unit: int8 layouts (Q8_0, Q6_K) 16, nibble layouts
// (Q4_0, Q4_K) 32, F32 4.
template <int QT>
constexpr int unit_floats() { return int8_layout(QT) ? 16 : (nibble_layout(QT) ? 32 : 4); }

// Load the input rows into LDS, times the RMSNorm gain when the prologue norm is
// on, and return each row's norm scale rsqrt(mean_k x^2 + eps) (1 without norm).
// The scale is a per-row scalar, so it is applied to the finished dot products
// (sum_k W[n][k] x[k] s w[k] = s * sum_k W[n][k] (x[k] w[k])); the staging is
// then one pass over x, with up to 8 float4 loads per thread in flight (no
// dependent round trip per element).  Rows mi >= a.m are zero.
// Layout: unit-transposed float4s, xs4[(mi * NV + i) * NU + u] holds floats
// 4i..4i+3 of unit u (NV float4 per unit, NU units per row).  A lane owns one
// unit, so for each slot i consecutive lanes read consecutive float4s: no bank
// conflicts (the natural layout puts every lane's unit 64 or 128 bytes apart,
// which lands all lanes on a handful of banks).
// issue(): called once, right after the loads of the first batch of inputs
// (before them with the residual prologue): the caller requests its first
// weight tiles there.  Loads return in order, so inputs requested behind the
// weight tiles could not be staged before those tiles arrive.
template <int QT, int M, int NW, bool RES, bool ACC, typename F>
QD_DEV void gemv_stage_x(const GemvArgs& a, float4* xs4, int kp, float (&scale)[M], F&& issue) {
  constexpr int NT = 64 * NW;  // threads of the workgroup
  constexpr int US = unit_floats<QT>(), NV = US / 4;
  // k positions per thread per batch (loads in flight); the residual prologue
  // loads four float4 per position, so it batches fewer to stay within the
  // register budget of the plain kernels (the weight tiles are live meanwhile).
  // Slots of a batch that start past the row are skipped as a whole (a
  // workgroup-uniform test), so short rows issue no extra loads.
  constexpr int JB = RES ? (M >= 2 ? 1 : 2) : (M >= 8 ? 1 : 8 / M);
  const int NU = kp / US, NK4 = kp / 4;
  [[maybe_unused]] float* xsum = reinterpret_cast<float*>(xs4 + M * NK4);  // nibble layouts: [M][nblk] block sums
  __shared__ float red[NW][M];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool norm = a.norm_w != nullptr;
  const float4* w4 = reinterpret_cast<const float4*>(a.norm_w);
  const int ldx4 = a.ldx / 4;
  float ss[M];
#pragma unroll
  for (int mi = 0; mi < M; ++mi) ss[mi] = 0.f;
  // residual prologue: the RMS scale of res_add first (one more pass over it)
  constexpr bool resid = RES;  // residual prologue (compiled only where used)
  const float4* t4 = reinterpret_cast<const float4*>(a.res_add);
  const float4* r4 = reinterpret_cast<const float4*>(a.res_w);
  float4* o4 = reinterpret_cast<float4*>(a.res_out);
  const bool write_h = resid && o4 && blockIdx.x == 0;
  float ts[M];
  if constexpr (RES) issue();
  if constexpr (RES) {
    __shared__ float red_t[NW][M];
#pragma unroll
    for (int mi = 0; mi < M; ++mi) ts[mi] = 0.f;
    for (int k0 = tid; k0 < NK4; k0 += NT * JB) {
      float4 tv[JB][M];
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int mi = 0; mi < M; ++mi)
          tv[j][mi] = (k0 + NT * j < NK4 && mi < a.m) ? t4[(size_t)mi * ldx4 + k0 + NT * j]
                                                      : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int mi = 0; mi < M; ++mi) {
          const float4 v = tv[j][mi];
          ts[mi] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
    }
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
      const float t = wave_sum(ts[mi]);
      if (lane == 0) red_t[wave][mi] = t;
    }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += red_t[w][mi];
      ts[mi] = 1.0f / sqrtf(t / (float)kp + a.eps);
    }
  }
  // one batch of JB positions per thread, from position b0 of the row (a
  // multiple of NT JB); the first batch is run by every thread, as
  // straight-line code, so that issue() is unconditional
  auto batch = [&](int b0, auto first) {
    float4 xv[JB][M], wv[JB];
    XRaw<ACC> xr[JB][M];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      if (b0 + NT * j >= NK4) break;  // the same for every thread
      const int k4 = b0 + NT * j + tid;
      const bool ok = k4 < NK4;
      if (norm) wv[j] = w4[ok ? k4 : 0];
#pragma unroll
      for (int mi = 0; mi < M; ++mi) xr[j][mi] = load_x4_raw<ACC>(a, mi, k4, ok);
    }
    if constexpr (decltype(first)::value && !RES) issue();
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      if (b0 + NT * j >= NK4) break;
      const int k4 = b0 + NT * j + tid;
      const bool ok = k4 < NK4;
      if (!(ok && norm)) wv[j] = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
      for (int mi = 0; mi < M; ++mi) xv[j][mi] = x4_value<ACC>(a, xr[j][mi], mi, ok);
      if constexpr (RES) {
        const float4 rw = ok ? r4[k4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int mi = 0; mi < M; ++mi) {
          const float4 t = (ok && mi < a.m) ? t4[(size_t)mi * ldx4 + k4] : make_float4(0.f, 0.f, 0.f, 0.f);
          const float s = ts[mi];
          xv[j][mi].x += t.x * s * rw.x;
          xv[j][mi].y += t.y * s * rw.y;
          xv[j][mi].z += t.z * s * rw.z;
          xv[j][mi].w += t.w * s * rw.w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      if (b0 + NT * j >= NK4) break;
      const int k4 = b0 + NT * j + tid;
      const bool ok = k4 < NK4;
      const int slot = (k4 % NV) * NU + k4 / NV;
#pragma unroll
      for (int mi = 0; mi < M; ++mi) {
        const float4 v = xv[j][mi], w = wv[j];
        const float4 p = make_float4(v.x * w.x, v.y * w.y, v.z * w.z, v.w * w.w);
        if (ok) {
          if (write_h && mi < a.m) o4[(size_t)mi * ldx4 + k4] = v;
          ss[mi] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          xs4[mi * NK4 + slot] = p;
        }
        if constexpr (nibble_layout(QT)) {
          // the block sums of the staged values: a block's eight float4 are
          // the k4 of eight consecutive lanes (NT and b0 are multiples of 64;
          // lanes past the row hold zeros and whole blocks, kp being a
          // multiple of 32); all lanes take part in the lane sums
          const float bsum = group_sum<8>(ok ? (p.x + p.y) + (p.z + p.w) : 0.f);
          if (ok && k4 % NV == 0) xsum[mi * (NK4 / NV) + k4 / NV] = bsum;
        }
      }
    }
  };
  batch(0, std::true_type{});
  for (int b0 = NT * JB; b0 < NK4; b0 += NT * JB) batch(b0, std::false_type{});
  if (norm) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
      const float t = wave_sum(ss[mi]);
      if (lane == 0) red[wave][mi] = t;
    }
  }
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < M; ++mi) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w][mi];
    scale[mi] = norm ? 1.0f / sqrtf(t / (float)kp + a.eps) : 1.f;
  }
}

// Weights of one row group held in registers between load and use.  Scales
// stay raw words until the tile is computed: converting them on arrival would
// make the wave wait for its newest loads right after issuing them.
template <int QT, int R, int U>
struct WRegs {
  uint4 w[R][U];
  uint32_t ks[R][U], kd[R][U];  // fp16 scale bits (Q8_0, Q4_0); K-quants: packed scale words
};

// Rows of group `grp`: R consecutive rows, or for the pair modes R/2 outputs,
// each a (gate, up) row pair of the interleaved layout.
template <int R, bool PAIR>
QD_DEV void group_rows(int grp, int rows, int (&r)[R]) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if constexpr (PAIR) {
      const int n = grp * (R / 2) + i / 2;
      r[i] = pair_gate_row(n) + (i & 1) * 32;
    } else {
      r[i] = min(grp * R + i, rows - 1);
    }
  }
}

// Issue the loads of U units per lane for R rows: unit u = base + lane + 64 k.
// Units past the row end are clamped to the last unit (a valid address, so the
// loads need no predicate); gemv_compute skips them.  Row bases are scalar and
// lane offsets unsigned 32-bit, so each load is a scalar base + vector offset.
// live = false (a tile past the wave's last one) points every lane's loads at
// the first bytes of `park`, the input row the workgroup has just read: one
// cache line per load, an L2 hit, no HBM bytes.  The loads are issued either
// way: with the same number of loads on every path through the ring, the
// compiler can wait for exactly the tile it is about to use instead of for all
// loads.
template <int QT, int R, int U>
QD_DEV void gemv_load(const GemvArgs& a, const int (&r)[R], int base, int lane, int nunits, WRegs<QT, R, U>& W,
                      bool live, const uint8_t* park) {
  const int kp = a.nblk * 32;
  auto at = [&](const void* p, size_t off) { return live ? static_cast<const uint8_t*>(p) + off : park; };
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const unsigned uc = live ? (unsigned)min(base + lane + 64 * k, nunits - 1) : 0u;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const size_t row = (size_t)r[i];
      if constexpr (QT == kQ8_0) {
        W.w[i][k] = load_nt(reinterpret_cast<const uint4*>(at(a.qs, row * kp) + uc * 16u));
        W.ks[i][k] = load_nt(reinterpret_cast<const uint16_t*>(at(a.d, row * a.nblk * 2)) + (uc >> 1));
      } else if constexpr (QT == kQ4_0) {
        W.w[i][k] = load_nt(reinterpret_cast<const uint4*>(at(a.qs, row * a.nblk * 16) + uc * 16u));
        W.ks[i][k] = load_nt(reinterpret_cast<const uint16_t*>(at(a.d, row * a.nblk * 2)) + uc);
      } else if constexpr (QT == kQ4_K) {
        W.w[i][k] = load_nt(reinterpret_cast<const uint4*>(at(a.qs, row * a.nblk * 16) + uc * 16u));
        W.ks[i][k] = load_nt(reinterpret_cast<const uint16_t*>(at(a.d, row * a.nblk * 2)) + uc);
        W.kd[i][k] = load_nt(reinterpret_cast<const uint32_t*>(at(a.sd, row * (a.nblk >> 3) * 4)) + (uc >> 3));
      } else if constexpr (QT == kQ6_K) {
        W.w[i][k] = load_nt(reinterpret_cast<const uint4*>(at(a.qs, row * kp) + uc * 16u));
        W.ks[i][k] = load_nt(reinterpret_cast<const int8_t*>(at(a.d, row * 2 * a.nblk)) + uc);
        W.kd[i][k] = load_nt(reinterpret_cast<const uint32_t*>(at(a.sd, row * (a.nblk >> 3) * 4)) + (uc >> 4));
      } else {
        W.w[i][k] = load_nt(reinterpret_cast<const uint4*>(at(a.qs, row * kp * 4) + uc * 16u));
      }
    }
  }
}

// One Q4_0 block given its 32 activations as 8 float4 (elements 0..15 in
// xv[0..3], 16..31 in xv[4..7]): 2^-24 * sum_j n_j x_j with the raw nibbles n
// (no offset).  Word i of the block holds elements 4i..4i+3 in its low nibbles
// and 4i+16..4i+19 in its high nibbles.  Masking a word with 0x000F000F leaves
// two nibbles in the low bits of its 16-bit halves, where they read as fp16
// subnormals n * 2^-24 (0x00F000F0: 16 n * 2^-24); the mixed-precision FMA
// takes an fp16 half directly (op_sel), so a weight costs one FMA plus 5/8 of
// a mask or shift, where a byte conversion would add a whole instruction.  The
// fp16 values are exact, and the power-of-two factor leaves every product and
// every rounding of the sums as for n x (f32 has the exponent range to spare;
// denormals are preserved), so the result is the f32 sum times 2^-24.
QD_DEV float dot32_q4_raw4(uint4 w, const float4 (&xv)[8]) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  float lo = 0.f, hi = 0.f;
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = words[i] >> 8;
    const h2 a = __builtin_bit_cast(h2, opaque_and(words[i], 0x000F000Fu));  // elements 4i, 4i+2
    const h2 c = __builtin_bit_cast(h2, opaque_and(s, 0x000F000Fu));         // 4i+1, 4i+3
    const h2 b = __builtin_bit_cast(h2, opaque_and(words[i], 0x00F000F0u));  // 4i+16, 4i+18 (x16)
    const h2 e = __builtin_bit_cast(h2, opaque_and(s, 0x00F000F0u));         // 4i+17, 4i+19 (x16)
    const float4 xl = xv[i], xh = xv[4 + i];
    lo = fmaf((float)a.x, xl.x, lo);
    lo = fmaf((float)c.x, xl.y, lo);
    lo = fmaf((float)a.y, xl.z, lo);
    lo = fmaf((float)c.y, xl.w, lo);
    hi = fmaf((float)b.x, xh.x, hi);
    hi = fmaf((float)e.x, xh.y, hi);
    hi = fmaf((float)b.y, xh.z, hi);
    hi = fmaf((float)e.y, xh.w, hi);
  }
  return lo + 0.0625f * hi;
}
constexpr float kTwo24 = 16777216.0f;

template <int QT, int R, int U, int M>
QD_DEV void gemv_compute(const float4* xs4, const float* xsum, int kp, int nblk, int base, int lane, int nunits,
                         const WRegs<QT, R, U>& W, float (&acc)[R][M]) {
  constexpr int NV = unit_floats<QT>() / 4;
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int u = base + lane + 64 * k;
    if (u >= nunits) continue;
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
      float4 xv[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) xv[i] = xs4[(mi * NV + i) * nunits + u];
      if constexpr (QT == kQ6_K) {
#pragma unroll
        for (int i = 0; i < R; ++i)
          acc[i][mi] += q6k_scale(W.ks[i][k], W.kd[i][k]) * dot16_q8(W.w[i][k], xv[0], xv[1], xv[2], xv[3]);
      } else if constexpr (QT == kQ8_0) {
#pragma unroll
        for (int i = 0; i < R; ++i)
          acc[i][mi] += half_bits_to_float((uint16_t)W.ks[i][k]) * dot16_q8(W.w[i][k], xv[0], xv[1], xv[2], xv[3]);
      } else if constexpr (QT == kQ4_0) {
        const float bs = 8.0f * xsum[mi * nblk + u];
#pragma unroll
        for (int i = 0; i < R; ++i)
          acc[i][mi] += half_bits_to_float((uint16_t)W.ks[i][k]) * fmaf(dot32_q4_raw4(W.w[i][k], xv), kTwo24, -bs);
      } else if constexpr (QT == kQ4_K) {
        const float xs = xsum[mi * nblk + u];
#pragma unroll
        for (int i = 0; i < R; ++i)
          acc[i][mi] += q4k_scale(W.ks[i][k], W.kd[i][k]) * (dot32_q4_raw4(W.w[i][k], xv) * kTwo24) -
                        q4k_min(W.ks[i][k], W.kd[i][k]) * xs;
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const uint4 w = W.w[i][k];
          acc[i][mi] += __uint_as_float(w.x) * xv[0].x + __uint_as_float(w.y) * xv[0].y +
                        __uint_as_float(w.z) * xv[0].z + __uint_as_float(w.w) * xv[0].w;
        }
      }
    }
  }
}

// Outputs of the wave's row groups are held in registers until the wave is
// done (obuf[mi], lane l = the l-th output of the wave) and written by one
// pass at the end: a store (or the residual add's load) inside the ring would
// make every later wait for a weight tile a wait for all loads in flight,
// since loads and stores share one in-order counter.
// Outputs per row group: R rows, or R / 2 (gate, up) pairs.
template <int MODE, int R>
constexpr int group_outputs() { return (MODE == kModePairSilu || MODE == kModePairGelu) ? R / 2 : R; }

// Finish a row group: reduce each accumulator over the 64 lanes, apply the
// input row's norm scale (and the pair activation), and put the group's
// outputs into lanes nslot.. of obuf.
template <int M, int MODE, int R>
QD_DEV void gemv_group_end(const float (&scale)[M], float (&acc)[R][M], float (&obuf)[M], int lane, int nslot) {
  constexpr bool kPair = MODE == kModePairSilu || MODE == kModePairGelu;
#pragma unroll
  for (int mi = 0; mi < M; ++mi) {
    if constexpr (R == 2) {
      // both rows in one lane tree: lanes of parity i hold row i's sum
      const float t = pair_wave_sum(acc[0][mi], acc[1][mi], lane) * scale[mi];
      float v;
      if constexpr (kPair) {  // (gate, up) = rows (0, 1); lane nslot takes the output
        const float u = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(t), 0xB1, 0xf, 0xf, true));
        const float gate = (lane & 1) ? u : t, up = (lane & 1) ? t : u;
        v = (MODE == kModePairSilu ? act_silu(gate) : act_gelu_tanh(gate)) * up;
        if (lane == nslot) obuf[mi] = v;
      } else {  // rows 0 and 1 into lanes nslot and nslot + 1 (nslot is even)
        if ((lane & ~1) == nslot) obuf[mi] = t;
      }
      acc[0][mi] = acc[1][mi] = 0.f;
      continue;
    }
    float sv[R];
#pragma unroll
    for (int i = 0; i < R; ++i) sv[i] = wave_sum(acc[i][mi]) * scale[mi];
#pragma unroll
    for (int j = 0; j < group_outputs<MODE, R>(); ++j) {
      float v;
      if constexpr (kPair) v = (MODE == kModePairSilu ? act_silu(sv[2 * j]) : act_gelu_tanh(sv[2 * j])) * sv[2 * j + 1];
      else v = sv[j];
      if (lane == nslot + j) obuf[mi] = v;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) acc[i][mi] = 0.f;
  }
}

// Write the nslot outputs held in obuf: lane l holds output j = l % RO of the
// wave's k-th row group, k = l / RO (row group gwave + k * nwaves), with the
// mode's epilogue (store: + bias; add: added to y).  AM: each lane keeps the
// best (value, index) it has written in bv / bi.
template <int M, int MODE, int R, bool AM>
QD_DEV void gemv_flush(const GemvArgs& a, float* ybase, int lane, int gwave, int nwaves, int nslot,
                       const float (&obuf)[M], float (&bv)[M], int (&bi)[M]) {
  constexpr int RO = group_outputs<MODE, R>();
  const int nout = (MODE == kModePairSilu || MODE == kModePairGelu) ? a.rows / 2 : a.rows;
  const int o = (gwave + (lane / RO) * nwaves) * RO + lane % RO;
  if (lane >= nslot || o >= nout) return;
#pragma unroll
  for (int mi = 0; mi < M; ++mi) {
    if (mi >= a.m) break;
    float* yr = ybase + (size_t)mi * a.ldy;
    float v = obuf[mi];
    if constexpr (MODE == kModeAdd) v = yr[o] + v;
    else if constexpr (MODE == kModeStore) v = a.bias ? v + a.bias[o] : v;
    yr[o] = v;
    if constexpr (AM) {
      if (ranks_before(v, o, bv[mi], bi[mi])) {
        bv[mi] = v;
        bi[mi] = o;
      }
    }
  }
}

// Register sets of the weight pipeline: with NS sets, NS - 1 tiles are in
// flight while one is computed.  Two sets for two-row tiles and three for
// one-row tiles: with one 16-byte unit per lane a deeper ring costs more in
// occupancy than it gains in loads in flight (measured on the decode shapes of
// the 0.6B and 8B models, one and sixteen input rows).
template <int R, int U, int M, int NW>
constexpr int gemv_sets() { return R * U == 1 ? 3 : 2; }

// R rows per wave, U 16-byte units per lane in flight per row, M input rows.
// Each wave walks its (row group, unit block) tiles in order through a ring of
// NS register sets: before tile t is computed, the loads of tile t + NS - 1 are
// issued into the set that tile t - 1 used, so NS - 1 tiles stay in flight
// through the arithmetic, the lane reduction and the store.  The first NS - 1
// tiles are requested before the input rows are staged.  Tile indices are
// wave-uniform (scalar registers), so every load is a scalar base plus a 32-bit
// lane offset.
template <int QT, int M, int MODE, int R, int U, int NW, bool RES, bool ACC = false, bool AM = false>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(GemvArgs a) {
  constexpr int NS = gemv_sets<R, U, M, NW>();
  extern __shared__ float4 xs4[];
  const int kp = a.nblk * 32;
  float* xsum = reinterpret_cast<float*>(xs4 + M * kp / 4);  // nibble layouts: [M][nblk] block sums of x
  constexpr bool kPair = MODE == kModePairSilu || MODE == kModePairGelu;
  const int lane = threadIdx.x & 63;
  const int gwave = __builtin_amdgcn_readfirstlane(blockIdx.x * NW + (threadIdx.x >> 6));
  const int nwaves = gridDim.x * NW;
  const int nunits = int8_layout(QT) ? 2 * a.nblk : (nibble_layout(QT) ? a.nblk : kp / 4);
  const int ngroups = kPair ? a.rows / R : (a.rows + R - 1) / R;
  const int tpg = (nunits + 64 * U - 1) / (64 * U);  // tiles per row group

  const uint8_t* const park = reinterpret_cast<const uint8_t*>(a.x ? a.x : a.xd);

  // Sets are always named by compile-time indices (integral_constant
  // arguments), so they stay in registers whether or not loops unroll.
  WRegs<QT, R, U> ws[NS];
  int tg[NS], tt[NS];  // (row group, tile within the group) held by each set
  int g = gwave, t = 0;  // next tile to request
  // request the tile (g, t) into set S and advance (g, t); past the wave's
  // last tile the set's loads are parked (see gemv_load)
  auto request = [&](auto S) {
    constexpr int s = decltype(S)::value;
    tg[s] = g;
    tt[s] = t;
    const bool live = g < ngroups;
    int r[R];
    group_rows<R, kPair>(live ? g : 0, a.rows, r);
    gemv_load<QT, R, U>(a, r, t * 64 * U, lane, nunits, ws[s], live, park);
    if (live && ++t == tpg) {
      t = 0;
      g += nwaves;
    }
  };
  float scale[M];
  // the first NS - 1 tiles are requested right behind the first input loads
  gemv_stage_x<QT, M, NW, RES, ACC>(a, xs4, kp, scale, [&] {
    request(std::integral_constant<int, 0>{});
    if constexpr (NS > 2) request(std::integral_constant<int, 1>{});
    if constexpr (NS > 3) request(std::integral_constant<int, 2>{});
  });  // ends with a barrier (the staged rows and, for nibble layouts, their block sums)

  float acc[R][M];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int mi = 0; mi < M; ++mi) acc[i][mi] = 0.f;
  float obuf[M];  // the wave's finished outputs, one per lane (gemv_group_end)
  float bv[M];    // AM: each lane's best written value and its row
  int bi[M];
#pragma unroll
  for (int mi = 0; mi < M; ++mi) {
    obuf[mi] = 0.f;
    bv[mi] = -INFINITY;
    bi[mi] = 0x7fffffff;
  }
  // the output rows, resolved once (y_ind: a pointer in device memory)
  float* const ybase = a.y_ind ? *a.y_ind + a.y_off : a.y;
  constexpr int RO = group_outputs<MODE, R>();
  int nslot = 0;  // outputs held in obuf (the launch gives a wave at most 64)

  // One ring step on set S: refill the set computed last (a parked load past
  // the wave's last tile), then compute S.  Every step that runs issues the
  // same loads, and the loop is left right after the wave's last tile, so no
  // path skips a step and then continues with the next one.
  auto step = [&](auto S) {
    constexpr int s = decltype(S)::value;
    request(std::integral_constant<int, (s + NS - 1) % NS>{});
    gemv_compute<QT, R, U, M>(xs4, xsum, kp, a.nblk, tt[s] * 64 * U, lane, nunits, ws[s], acc);
    if (tt[s] == tpg - 1) {
      gemv_group_end<M, MODE, R>(scale, acc, obuf, lane, nslot);
      nslot += RO;
    }
  };
  // the wave's tiles: row groups gwave, gwave + nwaves, ... below ngroups
  int left = gwave < ngroups ? ((ngroups - 1 - gwave) / nwaves + 1) * tpg : 0;
  static_assert(NS >= 2 && NS <= 4, "gemv: two to four register sets");
  while (left > 0) {
    step(std::integral_constant<int, 0>{});
    if (--left == 0) break;
    step(std::integral_constant<int, 1>{});
    if (--left == 0) break;
    if constexpr (NS > 2) {
      step(std::integral_constant<int, 2>{});
      if (--left == 0) break;
    }
    if constexpr (NS > 3) {
      step(std::integral_constant<int, 3>{});
      --left;
    }
  }
  gemv_flush<M, MODE, R, AM>(a, ybase, lane, gwave, nwaves, nslot, obuf, bv, bi);
  if constexpr (AM) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
      argmax_pair_wave(bv[mi], bi[mi]);
      if (lane == 0 && mi < a.m) {
        a.amax_v[(size_t)mi * nwaves + gwave] = bv[mi];
        a.amax_i[(size_t)mi * nwaves + gwave] = bi[mi];
      }
    }
  }
}

// ------------------------------------------------------------ batched decode on the matrix cores
// Decode projection of 5..16 input rows (a decode batch), Q4_0 / Q8_0 / Q4_K /
// Q6_K weights: y[m][n] = sum_k W[n][k] x[m][k] on V_MFMA_F32_16X16X4F32 (f32
// operands, f32 accumulation), with the weights decoded exactly in registers
// (dq_byte: d q for Q4_0 / Q8_0 / Q6_K, scale n - min for Q4_K, each rounded
// once as in the prefill GEMM) and the inputs read straight from global memory (no LDS
// staging, so rows of any length take all 16 inputs in one launch).  With the
// lane-tree GEMV, sixteen inputs cost two wave reductions per row and input
// and sixteen FMAs per weight on the vector ALU; here the matrix cores do the
// products and the sums over k.
//
// Workgroup = 16 outputs (pair modes: 16 (gate, up) pairs), four waves
// splitting K in groups of four quant blocks; blockIdx.y splits K further
// across ks = gridDim.y workgroups (wave w of workgroup z takes groups
// 4 z + w, 4 z + w + 4 ks, ...), for projections with few outputs, which then
// add their partial sums to y with atomic adds (add mode only: the order of
// the adds varies, so such outputs agree with themselves to f32 rounding).
// ACC: the input rows are decode attention's accumulators (the blocks summed
// and divided by their softmax denominators, as the lane-tree kernel's
// staging does), add mode only.  The add mode takes no norm prologue.
//
// Lane l = i + 16 q: weight row i and input row i of the tile, block q of the
// group.  The contraction index of MFMA step s is (block q, element s):
// lane (i, q) supplies A[i][q] = W[row i][(4g + q) 32 + s] and B[q][i] =
// x[i][(4g + q) 32 + s], so each lane reads one whole block of its row and 32
// consecutive inputs.  D[n][m] (output row n, input m) lands in register r of
// lane m + 16 (n / 4), r = n % 4.  The waves' partial tiles, and for the
// RMSNorm prologue the partial sums of squares, meet in LDS; wave 0 applies
// the norm scale (1 / rms, as the lane-tree kernel does: the gains multiply the
// inputs, the scale the sums) and the epilogue.
template <int QT, int MODE, bool ACC = false>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(GemvArgs a) {
  static_assert(QT == kQ4_0 || QT == kQ8_0 || QT == kQ4_K || QT == kQ6_K, "matrix-core decode: block-quantized types");
  constexpr bool kI8 = int8_layout(QT);  // 32 bytes per block (Q8_0, Q6_K), else 16 nibble bytes
  constexpr bool kKQ = QT == kQ4_K || QT == kQ6_K;  // scale words plus a super-block word
  static_assert(!ACC || MODE == kModeAdd, "accumulator input: add mode");
  constexpr bool kPair = MODE == kModePairSilu || MODE == kModePairGelu;
  constexpr bool kNorm = MODE != kModeAdd;  // the RMSNorm prologue (if norm_w is set)
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ f32x4 red[4][kPair ? 2 : 1][64];
  __shared__ float rss[4][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16;  // first output of the tile
  const int nout = kPair ? a.rows / 2 : a.rows;
  const int kp = a.nblk * 32;
  const int ngrp = (a.nblk + 3) / 4;
  const int ks = gridDim.y, kz = blockIdx.y;
  // weight rows of lane i (clamped into the matrix: rows past it are not stored)
  int row, row_up = 0;
  if constexpr (kPair) {
    row = pair_gate_row(min(n0 + i, nout - 1));
    row_up = row + 32;
  } else {
    row = min(n0 + i, a.rows - 1);
  }
  const bool xin = i < a.m;  // input row i exists
  const int mi = min(i, a.m - 1);
  const float* xrow = ACC ? a.xd + (size_t)mi * a.ldx : a.x + (size_t)mi * a.ldx;
  const bool norm = kNorm && a.norm_w != nullptr;
  const float* grow = norm ? a.norm_w : xrow;  // without a norm the row stands in, unused

  // ACC: g holds the second accumulator block, l the blocks' denominators
  struct Regs {
    uint4 w[kI8 ? 2 : 1], wu[kPair ? (kI8 ? 2 : 1) : 1];
    uint32_t d, du, sd, sdu;  // raw scale words; K-quants also their super-block words
    float4 x[8], g[kNorm || ACC ? 8 : 1];
    float l[ACC ? kAccCopies : 1];
  };
  static_assert(kAccCopies == 2, "two accumulator blocks");
  // loads of group g into R (every lane issues the same loads: blocks past
  // the row are read at the last block and zeroed when used)
  auto load = [&](int g, Regs& R) {
    const int kb = min(4 * g + q, a.nblk - 1);
    if constexpr (kI8) {
      const uint4* p = reinterpret_cast<const uint4*>(a.qs + (size_t)row * kp + kb * 32);
      R.w[0] = load_nt(p);
      R.w[1] = load_nt(p + 1);
      if constexpr (kPair) {
        const uint4* pu = reinterpret_cast<const uint4*>(a.qs + (size_t)row_up * kp + kb * 32);
        R.wu[0] = load_nt(pu);
        R.wu[1] = load_nt(pu + 1);
      }
    } else {
      R.w[0] = load_nt(reinterpret_cast<const uint4*>(a.qs + ((size_t)row * a.nblk + kb) * 16));
      if constexpr (kPair) R.wu[0] = load_nt(reinterpret_cast<const uint4*>(a.qs + ((size_t)row_up * a.nblk + kb) * 16));
    }
    R.d = load_nt(a.d + (size_t)row * a.nblk + kb);
    if constexpr (kPair) R.du = load_nt(a.d + (size_t)row_up * a.nblk + kb);
    if constexpr (kKQ) {
      R.sd = load_nt(a.sd + (size_t)row * (a.nblk >> 3) + (kb >> 3));
      if constexpr (kPair) R.sdu = load_nt(a.sd + (size_t)row_up * (a.nblk >> 3) + (kb >> 3));
    }
    const float4* xp = reinterpret_cast<const float4*>(xrow + kb * 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) R.x[e] = xp[e];
    if constexpr (ACC) {
      const float4* x2 = reinterpret_cast<const float4*>(xrow + a.xcstride + kb * 32);
#pragma unroll
      for (int e = 0; e < 8; ++e) R.g[e] = x2[e];
      // the block's 32 inputs lie in one head (head_dim a multiple of 32)
      const float* lp = a.xl + (size_t)mi * (a.ldx / a.xhd) + (kb * 32) / a.xhd;
      R.l[0] = lp[0];
      R.l[1] = lp[a.xcstride];
    } else if constexpr (kNorm) {
      const float4* gp = reinterpret_cast<const float4*>(grow + kb * 32);
#pragma unroll
      for (int e = 0; e < 8; ++e) R.g[e] = gp[e];
    }
  };
  // element s (0..31) of the lane's block, decoded: an int8 layout as
  // fma(d_s, q + 128, -128 d_s) = d_s q (d_s: the scale of element s's half of
  // the block, both halves alike but in Q6_K), a nibble layout as
  // fma(d, n, c) with c = -8 d (Q4_0) or -min (Q4_K); each rounds once
  auto weight = [&](const uint4 (&w)[kI8 ? 2 : 1], float d, float d2, float c, int s) -> float {
    if constexpr (kI8) {
      const uint32_t words[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
      const uint32_t u = words[s >> 2] ^ 0x80808080u;
      if (s >= 16) d = d2;
      const float cd = -128.f * d;
      switch (s & 3) {
        case 0: return dq_byte<0>(d, cd, u);
        case 1: return dq_byte<1>(d, cd, u);
        case 2: return dq_byte<2>(d, cd, u);
        default: return dq_byte<3>(d, cd, u);
      }
    } else {  // byte b: element b in its low nibble, b + 16 in its high one
      const uint32_t words[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
      const uint32_t wd = words[(s & 15) >> 2];
      const uint32_t u = s < 16 ? wd & 0x0f0f0f0fu : (wd >> 4) & 0x0f0f0f0fu;
      switch (s & 3) {
        case 0: return dq_byte<0>(d, c, u);
        case 1: return dq_byte<1>(d, c, u);
        case 2: return dq_byte<2>(d, c, u);
        default: return dq_byte<3>(d, c, u);
      }
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  auto compute = [&](int g, const Regs& R) {
    const bool ok = 4 * g + q < a.nblk;
    // a block past the row, or an input row past the batch, contributes
    // exact zeros (selects: its registers may hold anything)
    float d, d2, c, du = 0.f, du2 = 0.f, cu = 0.f;
    auto scales = [&](uint32_t dw, uint32_t sw, float& s0, float& s1, float& cc) {
      if constexpr (QT == kQ4_K) {
        s0 = s1 = q4k_scale(dw, sw);
        cc = -q4k_min(dw, sw);
      } else if constexpr (QT == kQ6_K) {
        s0 = q6k_scale((uint32_t)(int32_t)(int8_t)(dw & 0xffu), sw);
        s1 = q6k_scale((uint32_t)(int32_t)(int8_t)((dw >> 8) & 0xffu), sw);
        cc = 0.f;
      } else {
        s0 = s1 = half_bits_to_float((uint16_t)dw);
        cc = QT == kQ4_0 ? -8.f * s0 : 0.f;
      }
      if (!ok) s0 = s1 = cc = 0.f;
    };
    scales(R.d, kKQ ? R.sd : 0u, d, d2, c);
    if constexpr (kPair) scales(R.du, kKQ ? R.sdu : 0u, du, du2, cu);
    const bool use = ok && xin;
    float xs[32];
    if constexpr (ACC) {
      const float rl = 1.0f / (R.l[0] + R.l[1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 v = R.x[e], v2 = R.g[e];
        xs[4 * e + 0] = use ? (v.x + v2.x) * rl : 0.f;
        xs[4 * e + 1] = use ? (v.y + v2.y) * rl : 0.f;
        xs[4 * e + 2] = use ? (v.z + v2.z) * rl : 0.f;
        xs[4 * e + 3] = use ? (v.w + v2.w) * rl : 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 v = R.x[e], gg = R.g[kNorm ? e : 0];
        const float4 gv = (kNorm && norm) ? gg : make_float4(1.f, 1.f, 1.f, 1.f);
        xs[4 * e + 0] = use ? v.x * gv.x : 0.f;
        xs[4 * e + 1] = use ? v.y * gv.y : 0.f;
        xs[4 * e + 2] = use ? v.z * gv.z : 0.f;
        xs[4 * e + 3] = use ? v.w * gv.w : 0.f;
        if constexpr (kNorm) ss += use ? (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w) : 0.f;
      }
    }
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(weight(R.w, d, d2, c, s), xs[s], acc, 0, 0, 0);
      if constexpr (kPair)
        accu = __builtin_amdgcn_mfma_f32_16x16x4f32(weight(R.wu, du, du2, cu, s), xs[s], accu, 0, 0, 0);
    }
  };
  // two register sets: the wave's next group is requested before its
  // current one is computed
  Regs ra, rb;
  const int gs = 4 * ks;  // group stride of a wave
  int g = 4 * kz + wave;
  if (g < ngrp) load(g, ra);
  while (g < ngrp) {
    if (g + gs < ngrp) load(g + gs, rb);
    compute(g, ra);
    g += gs;
    if (g >= ngrp) break;
    if (g + gs < ngrp) load(g + gs, ra);
    compute(g, rb);
    g += gs;
  }
  red[wave][0][lane] = acc;
  if constexpr (kPair) red[wave][1][lane] = accu;
  rss[wave][lane] = ss;
  __syncthreads();
  if (wave != 0) return;
  f32x4 dsum = red[0][0][lane], usum = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kPair) usum = red[0][1][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    dsum += red[w][0][lane];
    if constexpr (kPair) usum += red[w][1][lane];
  }
  const int m = lane & 15;  // input row of this lane's outputs
  float scale = 1.f;
  if (norm) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) t += rss[w][m + 16 * qq];
    scale = 1.0f / sqrtf(t / (float)kp + a.eps);
  }
  if (m >= a.m) return;
  float* const yr = (a.y_ind ? *a.y_ind + a.y_off : a.y) + (size_t)m * a.ldy;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int n = n0 + 4 * q + r;
    if (n >= nout) continue;
    float v;
    if constexpr (kPair) {
      const float gt = dsum[r] * scale, up = usum[r] * scale;
      v = (MODE == kModePairSilu ? act_silu(gt) : act_gelu_tanh(gt)) * up;
    } else {
      v = dsum[r] * scale;
    }
    if constexpr (MODE == kModeAdd) {
      if (ks > 1) {
        unsafeAtomicAdd(yr + n, v);  // several workgroups add into this output
        continue;
      }
      v += yr[n];
    } else if constexpr (MODE == kModeStore) {
      v = a.bias ? v + a.bias[n] : v;
    }
    yr[n] = v;
  }
}

}  // namespace qd
