// Prefill projection: Y[t][n] = sum_k X[t][k] * W[n][k] for a whole prompt,
// W block-quantized in HBM -- a dense contraction, so it runs on the matrix
// cores (V_MFMA_F32_32X32X2_F32, f32 operands, f32 accumulation).
//
// Qwen3 walkthrough, "Overview" (prefill handles all prompt tokens at once) and
// Steps 5-6 (`x @ W.T` projections); Synsema "Choose the engine": weights stay
// quantized and are multiplied in f32.  Each weight tile is decoded exactly
// (d * q) into LDS as f32 once per workgroup and reused by all 64 token rows
// of the tile.
//
// Tiling: workgroup tile 64 tokens x 128 weight rows, BK = 32 (one quant block),
// LDS k-major (each MFMA operand read is 32 consecutive columns of one k row).
// Four waves in a 2 x 2 arrangement, each owning 32 tokens x 64 rows as two
// 32x32 accumulators.  MFMA lane layout (32x32x2 f32): A[i][k] from lane
// i + 32k, B[k][j] from lane j + 32k, D[i][j] in lane j + 32*((i/4)%2), register
// (i%4) + 4*(i/8).
#pragma once
#include "common.hpp"
#include "gemv.hpp"

namespace qd {

struct GemmArgs {
  const uint8_t* qs;    // weights, same layout as GemvArgs
  const uint16_t* d;
  int rows;
  int nblk;
  const float* x;       // [T][ldx]
  int ldx;
  int T;
  float* y;             // [T][ldy]
  int ldy;
  const uint32_t* sd;   // K-quant super-block scales (as GemvArgs)
};

template <int QT, int MODE>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a) {
  // Q4_0 / Q8_0 stage two quant blocks between barriers (their decode is two
  // instructions per value, so the staging stays cheap beside twice the
  // products; 48 KB of LDS): half the barriers per product, 0.74-0.80 of the
  // f32 MFMA peak on the 8B projections.  The other types stage one.
  constexpr int NBS = (QT == kQ8_0 || QT == kQ4_0) ? 2 : 1;
  constexpr int BM = 64, BN = 128, BK = 32 * NBS;
  // Columns XOR-swizzled within aligned 32-column blocks so that the staging
  // stores of a half-wave hit 32 distinct banks (X: four tokens x eight k
  // quads per half-wave; W: sixteen rows x the two k halves) while each MFMA
  // operand read stays a permutation of one aligned 32-column block:
  // X[t][k] at As[k][t ^ (k & 28)], W[n][k] at Bs[k][n ^ (16 * (bit 4 ^ bit 3 of k))].
  // One LDS stage: the next stage's global loads land in registers while the
  // current stage is multiplied, and a second barrier per stage guards the
  // overwrite (a second buffer only cost occupancy).
  __shared__ float As[BK][BM];
  __shared__ float Bs[BK][BN];
  auto sa = [](int k) { return k & 28; };
  auto sb = [](int k) { return (k ^ (k << 1)) & 16; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, t0 = blockIdx.y * BM;
  const int kp = a.nblk * 32;

  const int nst = (a.nblk + NBS - 1) / NBS;  // stages

  // staging registers
  float4 xa[2 * NBS];
  uint4 wq = make_uint4(0, 0, 0, 0);  // one-block types. int8 layouts: 16 int8; F32 uses wf[4]; nibble layouts the low 8 bytes
  // Q4_0 / Q8_0, block j of the stage.  Rows past the matrix never load: their
  // quant bytes and scale stay zero, which decodes to zeros without a select;
  // a stage's missing second block (odd block counts) gets scale zero.  The
  // scales stay raw fp16 bits until the stage is stored: converting them when
  // they are loaded would make the wave wait for its loads right there.
  uint4 wq2[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  uint32_t wh2[2] = {0u, 0u};
  bool wv2[2] = {false, false};
  float4 wf[4];
  float wd = 0.f, wmin = 0.f;  // block scale (Q6_K: of this thread's 16 values); Q4_K min
  uint32_t wks = 0, wkd = 0;   // K-quants: raw scale words, decoded when stored
  const int brow = tid >> 1, bhalf = tid & 1;
  const bool brow_ok = n0 + brow < a.rows;

  // X of stage kb, register i: block i / 2 of the stage, token row
  // (tid + 256 (i % 2)) / 8, k quad tid % 8 within the block (a half-wave
  // stores four tokens x eight quads of one block: the bank-free pattern)
  auto load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 2 * NBS; ++i) {
      const int idx = tid + 256 * (i & 1), row = idx >> 3, kq = (idx & 7) + 8 * (i >> 1);
      const int t = t0 + row;
      const bool ok = t < a.T && kb * NBS + (i >> 1) < a.nblk;
      xa[i] = ok ? *reinterpret_cast<const float4*>(a.x + (size_t)t * a.ldx + kb * BK + 4 * kq)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (brow_ok) {
      size_t r = n0 + brow;
      if constexpr (NBS == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int b = min(2 * kb + j, a.nblk - 1);  // a missing second block reads the last one, scaled by 0
          wh2[j] = a.d[r * a.nblk + b];
          wv2[j] = 2 * kb + j < a.nblk;
          if constexpr (QT == kQ8_0) {
            wq2[j] = *reinterpret_cast<const uint4*>(a.qs + r * kp + b * 32 + 16 * bhalf);
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(a.qs + (r * a.nblk + b) * 16 + 8 * bhalf);
            wq2[j].x = v.x;
            wq2[j].y = v.y;
          }
        }
      } else if constexpr (int8_layout(QT)) {
        wq = *reinterpret_cast<const uint4*>(a.qs + r * kp + kb * BK + 16 * bhalf);  // Q6_K
        wks = (uint32_t)(int32_t)reinterpret_cast<const int8_t*>(a.d)[r * 2 * a.nblk + 2 * kb + bhalf];
        wkd = a.sd[r * (a.nblk >> 3) + (kb >> 3)];
      } else if constexpr (nibble_layout(QT)) {  // Q4_K
        uint2 v = *reinterpret_cast<const uint2*>(a.qs + (r * a.nblk + kb) * 16 + 8 * bhalf);
        wq.x = v.x;
        wq.y = v.y;
        wks = a.d[r * a.nblk + kb];
        wkd = a.sd[r * (a.nblk >> 3) + (kb >> 3)];
      } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.qs) + r * kp + kb * BK + 16 * bhalf);
#pragma unroll
        for (int i = 0; i < 4; ++i) wf[i] = p[i];
      }
    }
  };

  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2 * NBS; ++i) {
      const int idx = tid + 256 * (i & 1), row = idx >> 3, kq = (idx & 7) + 8 * (i >> 1);
      As[4 * kq + 0][row ^ sa(4 * kq)] = xa[i].x;
      As[4 * kq + 1][row ^ sa(4 * kq + 1)] = xa[i].y;
      As[4 * kq + 2][row ^ sa(4 * kq + 2)] = xa[i].z;
      As[4 * kq + 3][row ^ sa(4 * kq + 3)] = xa[i].w;
    }
    if constexpr (QT == kQ4_K) {
      wd = q4k_scale(wks, wkd);
      wmin = q4k_min(wks, wkd);
    } else if constexpr (QT == kQ6_K) {
      wd = q6k_scale(wks, wkd);
    }
    if constexpr (QT == kQ8_0) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int k0 = 32 * jb + 16 * bhalf;  // block jb of the stage, this thread's half
        const uint32_t w4[4] = {wq2[jb].x, wq2[jb].y, wq2[jb].z, wq2[jb].w};
        const float d = wv2[jb] ? half_bits_to_float((uint16_t)wh2[jb]) : 0.f, cd = -128.f * d;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t u = w4[j] ^ 0x80808080u;
          Bs[k0 + 4 * j + 0][brow ^ sb(k0 + 4 * j + 0)] = dq_byte<0>(d, cd, u);
          Bs[k0 + 4 * j + 1][brow ^ sb(k0 + 4 * j + 1)] = dq_byte<1>(d, cd, u);
          Bs[k0 + 4 * j + 2][brow ^ sb(k0 + 4 * j + 2)] = dq_byte<2>(d, cd, u);
          Bs[k0 + 4 * j + 3][brow ^ sb(k0 + 4 * j + 3)] = dq_byte<3>(d, cd, u);
        }
      }
    } else if constexpr (QT == kQ4_0) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int k0 = 32 * jb + 8 * bhalf;  // block jb, this thread's eight bytes (low nibbles k0.., high k0 + 16..)
        const uint32_t w2[2] = {wq2[jb].x, wq2[jb].y};
        const float d = wv2[jb] ? half_bits_to_float((uint16_t)wh2[jb]) : 0.f, cd = -8.f * d;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t lo = w2[j] & 0x0f0f0f0fu, hi = (w2[j] >> 4) & 0x0f0f0f0fu;
          const int i = k0 + 4 * j;
          Bs[i + 0][brow ^ sb(i + 0)] = dq_byte<0>(d, cd, lo);
          Bs[i + 1][brow ^ sb(i + 1)] = dq_byte<1>(d, cd, lo);
          Bs[i + 2][brow ^ sb(i + 2)] = dq_byte<2>(d, cd, lo);
          Bs[i + 3][brow ^ sb(i + 3)] = dq_byte<3>(d, cd, lo);
          Bs[i + 16][brow ^ sb(i + 16)] = dq_byte<0>(d, cd, hi);
          Bs[i + 17][brow ^ sb(i + 17)] = dq_byte<1>(d, cd, hi);
          Bs[i + 18][brow ^ sb(i + 18)] = dq_byte<2>(d, cd, hi);
          Bs[i + 19][brow ^ sb(i + 19)] = dq_byte<3>(d, cd, hi);
        }
      }
    } else if constexpr (int8_layout(QT)) {
      uint32_t w4[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = brow_ok ? wd * (float)(int8_t)(w4[i >> 2] >> (8 * (i & 3))) : 0.f;
        Bs[16 * bhalf + i][brow ^ sb(16 * bhalf + i)] = v;
      }
    } else if constexpr (nibble_layout(QT)) {
      uint32_t w2[2] = {wq.x, wq.y};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t byte = (w2[i >> 2] >> (8 * (i & 3))) & 0xffu;
        // Q4_K: scale * n - min, rounded once
        float lo = fmaf(wd, (float)(byte & 15u), -wmin);
        float hi = fmaf(wd, (float)(byte >> 4), -wmin);
        lo = brow_ok ? lo : 0.f;
        hi = brow_ok ? hi : 0.f;
        Bs[8 * bhalf + i][brow ^ sb(8 * bhalf + i)] = lo;
        Bs[16 + 8 * bhalf + i][brow ^ sb(16 + 8 * bhalf + i)] = hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Bs[16 * bhalf + 4 * i + 0][brow ^ sb(16 * bhalf + 4 * i + 0)] = brow_ok ? wf[i].x : 0.f;
        Bs[16 * bhalf + 4 * i + 1][brow ^ sb(16 * bhalf + 4 * i + 1)] = brow_ok ? wf[i].y : 0.f;
        Bs[16 * bhalf + 4 * i + 2][brow ^ sb(16 * bhalf + 4 * i + 2)] = brow_ok ? wf[i].z : 0.f;
        Bs[16 * bhalf + 4 * i + 3][brow ^ sb(16 * bhalf + 4 * i + 3)] = brow_ok ? wf[i].w : 0.f;
      }
    }
  };

  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;

  load(0);
  store();
  __syncthreads();
  const int li = lane & 31, lk = lane >> 5;
  for (int kb = 0; kb < nst; ++kb) {
    if (kb + 1 < nst) load(kb + 1);
#pragma unroll
    for (int p = 0; p < BK / 2; ++p) {
      const int k = 2 * p + lk;
      float av = As[k][(wm * 32 + li) ^ sa(k)];
      float b0 = Bs[k][(wn * 64 + li) ^ sb(k)];
      float b1 = Bs[k][(wn * 64 + 32 + li) ^ sb(k)];
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1, acc1, 0, 0, 0);
    }
    __syncthreads();  // every wave is done reading the stage
    if (kb + 1 < nst) store();
    __syncthreads();
  }

  constexpr bool kPair = MODE == kModePairSilu || MODE == kModePairGelu;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    int i = 8 * (r >> 2) + 4 * lk + (r & 3);
    int t = t0 + wm * 32 + i;
    if (t >= a.T) continue;
    float* yr = a.y + (size_t)t * a.ldy;
    int n = n0 + wn * 64 + li;
    if constexpr (kPair) {
      int nn = (n0 + wn * 64) / 2 + li;
      if (n + 32 < a.rows) {
        float g = acc0[r], u = acc1[r];
        yr[nn] = (MODE == kModePairSilu ? act_silu(g) : act_gelu_tanh(g)) * u;
      }
    } else if constexpr (MODE == kModeAdd) {
      if (n < a.rows) yr[n] += acc0[r];
      if (n + 32 < a.rows) yr[n + 32] += acc1[r];
    } else {
      if (n < a.rows) yr[n] = acc0[r];
      if (n + 32 < a.rows) yr[n + 32] = acc1[r];
    }
  }
}

// Small-N variant: workgroup tile 32 tokens x 64 weight rows, NWV waves (4 or
// 8), BK = 32 NWV (one quant block per wave per stage).  Each wave owns its
// block of the stage over the whole 32 x 64 tile (two 32x32 accumulators),
// i.e. the waves split K; at the end the NWV partial tiles are summed through
// LDS in wave order (deterministic).  Four times the workgroups of the
// 64 x 128 tile for the same problem, for projections with few output rows (O
// and down at small hidden sizes, gate/up of short prompts); eight waves when
// even that grid leaves a CU with one workgroup.
template <int QT, int MODE, int NWV>
__global__ __launch_bounds__(64 * NWV, 1) void gemm_ksplit_kernel(GemmArgs a) {
  static_assert(NWV == 4 || NWV == 8, "four or eight waves");
  constexpr int BM = 32, BN = 64, BK = 32 * NWV, NT = 64 * NWV;
  // LDS k-major without padding; columns XOR-swizzled so that both the staging
  // writes and the MFMA operand reads of a half-wave hit 32 distinct banks:
  // X[t][k] at As[k][t ^ ((k / 4) % 32)], W[n][k] at Bs[k][n ^ (32 / NWV) (k / 32)].
  // One LDS stage, as in gemm_kernel.
  __shared__ float As[BK][BM];
  __shared__ float Bs[BK][BN];
  constexpr int SW = 32 / NWV;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * BN, t0 = blockIdx.y * BM;
  const int kp = a.nblk * 32;
  const int nstage = (a.nblk + NWV - 1) / NWV;

  // staging: X 32 rows x BK k = 8 NWV float4 per row, 4 per thread; W 64 rows
  // x NWV blocks (thread -> row tid / NWV, block tid % NWV: one quant block,
  // 32 weights)
  float4 xa[4];
  uint4 wq[2];
  float4 wf[8];
  float wd = 0.f, wd2 = 0.f, wmin = 0.f;  // scale (Q6_K: of values 0..15, wd2 of 16..31); Q4_K min
  uint32_t wks = 0, wkd = 0;              // raw scale words (Q4_0 / Q8_0: the fp16 bits), decoded when stored
  const int brow = tid / NWV, bblk = tid % NWV;
  const bool brow_ok = n0 + brow < a.rows;

  auto load = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i, row = idx / (BK / 4), kq = idx % (BK / 4);
      const int t = t0 + row, k = st * BK + 4 * kq;
      xa[i] = (t < a.T && k < kp) ? *reinterpret_cast<const float4*>(a.x + (size_t)t * a.ldx + k)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int kb = st * NWV + bblk;
    if (brow_ok && kb < a.nblk) {
      const size_t r = n0 + brow;
      if constexpr (int8_layout(QT)) {
        const uint4* p = reinterpret_cast<const uint4*>(a.qs + r * kp + kb * 32);
        wq[0] = p[0];
        wq[1] = p[1];
        if constexpr (QT == kQ8_0) {
          wks = a.d[r * a.nblk + kb];
        } else {  // the two int8 scales of the block's 16-value halves
          wks = a.d[r * a.nblk + kb];
          wkd = a.sd[r * (a.nblk >> 3) + (kb >> 3)];
        }
      } else if constexpr (nibble_layout(QT)) {
        wq[0] = *reinterpret_cast<const uint4*>(a.qs + (r * a.nblk + kb) * 16);
        wks = a.d[r * a.nblk + kb];
        if constexpr (QT == kQ4_K) wkd = a.sd[r * (a.nblk >> 3) + (kb >> 3)];
      } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.qs) + r * kp + kb * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) wf[i] = p[i];
      }
    } else {
      wq[0] = wq[1] = make_uint4(0, 0, 0, 0);
      wd = wd2 = wmin = 0.f;
      wks = wkd = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) wf[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i, row = idx / (BK / 4), kq = idx % (BK / 4);
      const int c = row ^ (kq & 31);
      As[4 * kq + 0][c] = xa[i].x;
      As[4 * kq + 1][c] = xa[i].y;
      As[4 * kq + 2][c] = xa[i].z;
      As[4 * kq + 3][c] = xa[i].w;
    }
    const int kk = bblk * 32, bc = brow ^ (SW * bblk);
    if constexpr (QT == kQ8_0 || QT == kQ4_0) {
      wd = half_bits_to_float((uint16_t)wks);  // zero bits (rows or blocks past the matrix): 0
    } else if constexpr (QT == kQ4_K) {
      wd = q4k_scale(wks, wkd);
      wmin = q4k_min(wks, wkd);
    } else if constexpr (QT == kQ6_K) {
      wd = q6k_scale((uint32_t)(int32_t)(int8_t)(wks & 0xffu), wkd);
      wd2 = q6k_scale((uint32_t)(int32_t)(int8_t)(wks >> 8), wkd);
    }
    if constexpr (QT == kQ8_0) {
      const uint32_t w8[8] = {wq[0].x, wq[0].y, wq[0].z, wq[0].w, wq[1].x, wq[1].y, wq[1].z, wq[1].w};
      const float cd = -128.f * wd;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t u = w8[j] ^ 0x80808080u;
        Bs[kk + 4 * j + 0][bc] = dq_byte<0>(wd, cd, u);
        Bs[kk + 4 * j + 1][bc] = dq_byte<1>(wd, cd, u);
        Bs[kk + 4 * j + 2][bc] = dq_byte<2>(wd, cd, u);
        Bs[kk + 4 * j + 3][bc] = dq_byte<3>(wd, cd, u);
      }
    } else if constexpr (int8_layout(QT)) {
      const uint32_t w8[8] = {wq[0].x, wq[0].y, wq[0].z, wq[0].w, wq[1].x, wq[1].y, wq[1].z, wq[1].w};
#pragma unroll
      for (int i = 0; i < 32; ++i)
        Bs[kk + i][bc] = (i < 16 ? wd : wd2) * (float)(int8_t)(w8[i >> 2] >> (8 * (i & 3)));
    } else if constexpr (QT == kQ4_K) {
      const uint32_t w4[4] = {wq[0].x, wq[0].y, wq[0].z, wq[0].w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t byte = (w4[i >> 2] >> (8 * (i & 3))) & 0xffu;
        Bs[kk + i][bc] = fmaf(wd, (float)(byte & 15u), -wmin);
        Bs[kk + 16 + i][bc] = fmaf(wd, (float)(byte >> 4), -wmin);
      }
    } else if constexpr (QT == kQ4_0) {
      const uint32_t w4[4] = {wq[0].x, wq[0].y, wq[0].z, wq[0].w};
      const float cd = -8.f * wd;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = w4[j] & 0x0f0f0f0fu, hi = (w4[j] >> 4) & 0x0f0f0f0fu;
        Bs[kk + 4 * j + 0][bc] = dq_byte<0>(wd, cd, lo);
        Bs[kk + 4 * j + 1][bc] = dq_byte<1>(wd, cd, lo);
        Bs[kk + 4 * j + 2][bc] = dq_byte<2>(wd, cd, lo);
        Bs[kk + 4 * j + 3][bc] = dq_byte<3>(wd, cd, lo);
        Bs[kk + 16 + 4 * j + 0][bc] = dq_byte<0>(wd, cd, hi);
        Bs[kk + 16 + 4 * j + 1][bc] = dq_byte<1>(wd, cd, hi);
        Bs[kk + 16 + 4 * j + 2][bc] = dq_byte<2>(wd, cd, hi);
        Bs[kk + 16 + 4 * j + 3][bc] = dq_byte<3>(wd, cd, hi);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Bs[kk + 4 * i + 0][bc] = wf[i].x;
        Bs[kk + 4 * i + 1][bc] = wf[i].y;
        Bs[kk + 4 * i + 2][bc] = wf[i].z;
        Bs[kk + 4 * i + 3][bc] = wf[i].w;
      }
    }
  };

  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
  load(0);
  store();
  __syncthreads();
  const int li = lane & 31, lk = lane >> 5;
  for (int st = 0; st < nstage; ++st) {
    if (st + 1 < nstage) load(st + 1);
    const int kw = wave * 32;  // this wave's quant block within the stage
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int k = kw + 2 * p + lk;
      const float av = As[k][li ^ ((k >> 2) & 31)];
      const float b0 = Bs[k][li ^ (SW * wave)];
      const float b1 = Bs[k][32 + (li ^ (SW * wave))];
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1, acc1, 0, 0, 0);
    }
    __syncthreads();  // every wave is done reading the stage
    if (st + 1 < nstage) store();
    __syncthreads();
  }
  // sum the waves' partial tiles in wave order (reusing the B buffer)
  static_assert(sizeof(Bs) >= NWV * BM * BN * sizeof(float), "reduction buffer");
  float* red = &Bs[0][0];  // NWV x [32][64] floats
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * lk + (r & 3);
    red[(wave * BM + i) * BN + li] = acc0[r];
    red[(wave * BM + i) * BN + 32 + li] = acc1[r];
  }
  __syncthreads();
  auto sum_waves = [&](int i, int j) {
    float v = red[i * BN + j];
#pragma unroll
    for (int w = 1; w < NWV; ++w) v += red[(w * BM + i) * BN + j];
    return v;
  };
  if constexpr (MODE == kModePairSilu || MODE == kModePairGelu) {
    // the tile's 64 rows are one (gate 32, up 32) group of the interleaved
    // layout: outputs n0 / 2 + j, j < 32
    for (int e = tid; e < BM * 32; e += NT) {
      const int i = e / 32, j = e % 32;
      const int t = t0 + i;
      if (t < a.T && n0 + j + 32 < a.rows) {
        const float g = sum_waves(i, j), u = sum_waves(i, j + 32);
        a.y[(size_t)t * a.ldy + n0 / 2 + j] = (MODE == kModePairSilu ? act_silu(g) : act_gelu_tanh(g)) * u;
      }
    }
  } else {
    for (int e = tid; e < BM * BN; e += NT) {
      const int i = e / BN, j = e % BN;
      const int t = t0 + i, n = n0 + j;
      if (t < a.T && n < a.rows) {
        const float v = sum_waves(i, j);
        float* yr = a.y + (size_t)t * a.ldy;
        if constexpr (MODE == kModeAdd) yr[n] += v;
        else yr[n] = v;
      }
    }
  }
}

// bf16-operand variant (Q8_0 / Q4_0 weights).  Quant values are small integers,
// exact in bf16; the block scale d stays f32 and multiplies each block's
// partial sums.  Activations are split into NT bf16 terms, x = x1 + x2 + x3
// with x1 = bf16(x), x2 = bf16(x - x1), x3 = x - x1 - x2 (NT = 3: exact, since
// f32 has 24 significant bits and each term takes 8; every product q * x_t is
// exact in the f32 accumulator, so the path is the f32 product up to summation
// order), or x ~ x1 (NT = 1: plain bf16 rounding of the activations).
// V_MFMA_F32_32X32X16_BF16: A[i][k] from lane i + 32 (k / 8), element k % 8;
// B[k][j] from lane j + 32 (k / 8); D as in the f32 32x32 forms.
// Tile 64 tokens x 128 rows, BK = 32 (one quant block), four waves 2 x 2, each
// 32 tokens x 64 rows: per block a wave issues 2 x NT x 2 MFMAs into a block
// accumulator, then adds d * (block accumulator) into its f32 result.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

QD_DEV void split_bf16(float x, __bf16 (&t)[3]) {
  t[0] = (__bf16)x;
  const float r = x - (float)t[0];
  t[1] = (__bf16)r;
  t[2] = (__bf16)(r - (float)t[1]);
}

template <int QT, int MODE, int NT>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BM = 64, BN = 128, BK = 32;
  constexpr int RS = BK + 8;  // row stride in bf16 (80 bytes): conflict-free 16-byte reads
  __shared__ __align__(16) __bf16 As[2][NT][BM][RS];
  __shared__ __align__(16) __bf16 Bs[2][BN][RS];
  __shared__ float Ds[2][BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, t0 = blockIdx.y * BM;
  const int kp = a.nblk * 32;

  // staging: X row tid / 4, k (tid % 4) * 8 .. +8; W row tid / 2, k (tid % 2) * 16 .. +16
  float4 xa[2];
  uint4 wq;
  uint32_t wh = 0u;  // the block's fp16 scale bits, converted when stored
  const int xrow = tid >> 2, xk = (tid & 3) * 8;
  const int brow = tid >> 1, bhalf = tid & 1;
  const bool brow_ok = n0 + brow < a.rows;

  auto load = [&](int kb) {
    const int t = t0 + xrow;
    if (t < a.T) {
      const float4* p = reinterpret_cast<const float4*>(a.x + (size_t)t * a.ldx + kb * BK + xk);
      xa[0] = p[0];
      xa[1] = p[1];
    } else {
      xa[0] = xa[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (brow_ok) {
      const size_t r = n0 + brow;
      if constexpr (QT == kQ8_0) wq = *reinterpret_cast<const uint4*>(a.qs + r * kp + kb * BK + 16 * bhalf);
      else wq = *reinterpret_cast<const uint4*>(a.qs + (r * a.nblk + kb) * 16);
      wh = a.d[r * a.nblk + kb];
    } else {
      wq = make_uint4(0, 0, 0, 0);
      wh = 0u;
    }
  };

  auto store = [&](int buf) {
    const float xv[8] = {xa[0].x, xa[0].y, xa[0].z, xa[0].w, xa[1].x, xa[1].y, xa[1].z, xa[1].w};
    bf16x8 xt[NT];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 t3[3];
      split_bf16(xv[e], t3);
#pragma unroll
      for (int t = 0; t < NT; ++t) xt[t][e] = t3[t];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<bf16x8*>(&As[buf][t][xrow][xk]) = xt[t];
    const uint32_t w4[4] = {wq.x, wq.y, wq.z, wq.w};
    bf16x8 q0, q1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v;
      if constexpr (QT == kQ8_0) {
        v = (float)(int8_t)(w4[e >> 2] >> (8 * (e & 3)));
      } else {
        const uint32_t byte = (w4[e >> 2] >> (8 * (e & 3))) & 0xffu;
        v = (float)((int)(bhalf ? (byte >> 4) : (byte & 15u)) - 8);
      }
      if (e < 8) q0[e] = (__bf16)v;
      else q1[e - 8] = (__bf16)v;
    }
    if (!brow_ok) q0 = q1 = bf16x8{};
    *reinterpret_cast<bf16x8*>(&Bs[buf][brow][16 * bhalf]) = q0;
    *reinterpret_cast<bf16x8*>(&Bs[buf][brow][16 * bhalf + 8]) = q1;
    if (bhalf == 0) Ds[buf][brow] = half_bits_to_float((uint16_t)wh);
  };

  f32x16 acc[2], blk[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s][r] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  const int li = lane & 31, kg = (lane >> 5) * 8;
  for (int kb = 0; kb < a.nblk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < a.nblk) load(kb + 1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) blk[s][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 bv[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) bv[s] = *reinterpret_cast<const bf16x8*>(&Bs[buf][wn * 64 + s * 32 + li][kk + kg]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&As[buf][t][wm * 32 + li][kk + kg]);
#pragma unroll
        for (int s = 0; s < 2; ++s) blk[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[s], blk[s], 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float d = Ds[buf][wn * 64 + s * 32 + li];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][r] += d * blk[s][r];
    }
    if (kb + 1 < a.nblk) store(buf ^ 1);
    __syncthreads();
  }

  constexpr bool kPair = MODE == kModePairSilu || MODE == kModePairGelu;
  const int lk = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * lk + (r & 3);
    const int t = t0 + wm * 32 + i;
    if (t >= a.T) continue;
    float* yr = a.y + (size_t)t * a.ldy;
    const int n = n0 + wn * 64 + li;
    if constexpr (kPair) {
      const int nn = (n0 + wn * 64) / 2 + li;
      if (n + 32 < a.rows) {
        const float g = acc[0][r], u = acc[1][r];
        yr[nn] = (MODE == kModePairSilu ? act_silu(g) : act_gelu_tanh(g)) * u;
      }
    } else if constexpr (MODE == kModeAdd) {
      if (n < a.rows) yr[n] += acc[0][r];
      if (n + 32 < a.rows) yr[n + 32] += acc[1][r];
    } else {
      if (n < a.rows) yr[n] = acc[0][r];
      if (n + 32 < a.rows) yr[n + 32] = acc[1][r];
    }
  }
}

}  // namespace qd
