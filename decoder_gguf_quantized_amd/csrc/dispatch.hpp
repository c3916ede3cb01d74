// Kernel dispatch: from run-time shapes to the template instantiations of the
// GEMV and GEMM kernels.  The instantiations of each weight type are compiled
// in a translation unit of their own (kern_<type>.hip), in parallel; the
// runtime (qdec.hip) calls them through gemv_launch<QT> / gemm_launch<QT>.
#pragma once
#include <hip/hip_runtime.h>

#include <string>

#include "common.hpp"
#include "gemm.hpp"
#include "gemv.hpp"

namespace qd {

// A HIP error or a broken invariant found while enqueueing; the C ABI turns it
// into status 2 and poisons the handle.
struct HipError {
  std::string msg;
};

template <typename... KArgs, typename... Args>
void qlaunch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st, Args... args) {
  // dynamic LDS beyond 64 KB (up to the CU's 160 KB) must be allowed per kernel
  if (lds > 64 * 1024) {
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) throw HipError{std::string("hipFuncSetAttribute: ") + hipGetErrorString(e)};
  }
  hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

// ------------------------------------------------------------ GEMV
// Modes of a tile class: PAIRC = the gate/up pair modes (SiLU or gelu_tanh,
// with or without the residual prologue); otherwise store and add, the
// residual prologue (store), the attention-accumulator input (store, add) and
// the fused argmax (store, one input row).
template <int QT, int M, int R, int U, int NW, bool PAIRC>
void gemv_dispatch_mode(int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  const unsigned nt = 64 * NW;
  if constexpr (PAIRC) {
    if (mode != kModePairSilu && mode != kModePairGelu) throw HipError{"gemv: a pair tile class needs a pair mode"};
    if (a.xd || a.amax_v) throw HipError{"gemv: pair modes take a plain input row"};
    const bool silu = mode == kModePairSilu;
    if (a.res_add) {
      if (silu) qlaunch(gemv_kernel<QT, M, kModePairSilu, R, U, NW, true>, grid, nt, lds, st, a);
      else qlaunch(gemv_kernel<QT, M, kModePairGelu, R, U, NW, true>, grid, nt, lds, st, a);
    } else {
      if (silu) qlaunch(gemv_kernel<QT, M, kModePairSilu, R, U, NW, false>, grid, nt, lds, st, a);
      else qlaunch(gemv_kernel<QT, M, kModePairGelu, R, U, NW, false>, grid, nt, lds, st, a);
    }
  } else {
    if (mode != kModeStore && mode != kModeAdd) throw HipError{"gemv: a row tile class needs store or add"};
    const bool add = mode == kModeAdd;
    if (a.amax_v) {  // the LM head of one row with the greedy choice in its epilogue
      if constexpr (M == 1) {
        if (add || a.xd) throw HipError{"gemv: the fused argmax needs the plain store epilogue"};
        if (a.res_add) qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, true, false, true>, grid, nt, lds, st, a);
        else qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, false, false, true>, grid, nt, lds, st, a);
      } else {
        throw HipError{"gemv: the fused argmax takes one input row"};
      }
    } else if (a.res_add) {  // residual prologue (sandwich norms)
      if (add || a.xd) throw HipError{"gemv: the residual prologue needs the store epilogue"};
      qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, true>, grid, nt, lds, st, a);
    } else if (a.xd) {  // input from decode attention's accumulators
      if (add) qlaunch(gemv_kernel<QT, M, kModeAdd, R, U, NW, false, true>, grid, nt, lds, st, a);
      else qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, false, true>, grid, nt, lds, st, a);
    } else {
      if (add) qlaunch(gemv_kernel<QT, M, kModeAdd, R, U, NW, false>, grid, nt, lds, st, a);
      else qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, false>, grid, nt, lds, st, a);
    }
  }
}

// Tile classes.  Every class gives a lane one 16-byte unit per row and tile
// (U = 1): small tiles spread each wave's arithmetic over the stream, which
// measured faster than two or four units per lane on every decode shape of
// the 0.6B and 8B models.  Eight-wave workgroups halve the input staging per
// CU, which pays on long rows (the 8B down projection 12.4 -> 10.1 us) but not
// for the gate/up pairs.
//   0: one row per wave, four-wave workgroups (store / add on fewer than 4,096
//      rows: two-row groups would leave CUs without a workgroup);
//   1: two rows per wave, eight-wave workgroups (store / add, 4,096 rows or
//      more);
//   2: one gate/up pair per wave, four-wave workgroups (pair modes, up to
//      four input rows);
//   3: two gate/up pairs per wave, four-wave workgroups (pair modes, eight or
//      sixteen input rows);
//   4: one row per wave, sixteen-wave workgroups (one input row, store / add,
//      4,096 rows or more, rows of 8,192 inputs or more): a CU stages the long
//      input row once for twice the waves of class 1 (the 8B down projection
//      10.1 -> 9.4 us; the same shape for the gate/up pairs, which are bound
//      by their vector arithmetic, measured 13.5 -> 15.6 us).
// LDS budget of the GEMV's staged input rows (the CU has 160 KB; the rest is
// left for the kernel's own small arrays).
constexpr size_t kGemvLdsMax = 128 * 1024;

// Tile class of the matrix-core decode (gemv_mfma_kernel), launched as
// M = 16 with one workgroup per 16 outputs (times the K split) and no LDS
// staging.  It takes 5..16 input rows of block-quantized weights (its cost does
// not depend on the row count; on the batched 0.6B-shape workload it measured
// 2,058 against 1,978 tokens/s at 8 sequences and 1,604 against 1,737 at 4):
//   - store and pair modes with plain inputs and at least 2,048 outputs: with
//     fewer, most CUs get no workgroup (the 0.6B-shape down projection, 1,024
//     outputs on 64 workgroups, took 17.6 us against 16.8 us for two eight-row
//     launches of the lane-tree kernel);
//   - the add mode without a norm prologue, plain or from decode attention's
//     accumulators, with K split across workgroups until there are about 256.
constexpr int kGemvMfmaClass = 8;
constexpr int kGemvMfmaMinRows = 5;
// the K split of the matrix-core decode for a projection (0: not taken)
inline int gemv_mfma_split(int type, int rows_in, int mode, int nout, int nblk, bool norm, bool res, bool acc,
                           bool amax) {
  if (type == kF32 || rows_in < kGemvMfmaMinRows || rows_in > 16 || res || amax) return 0;
  if (mode != kModeAdd) return (!acc && nout >= 2048) ? 1 : 0;
  if (norm) return 0;
  const int tiles = (nout + 15) / 16, ngrp = (nblk + 3) / 4;
  int ks = 1;
  while (tiles * ks < 256 && 4 * (ks + 1) <= ngrp) ++ks;  // each wave keeps a group at least
  return ks;
}

// plain: no residual prologue, no attention-accumulator input, no fused argmax
inline int gemv_tile_class(bool pair, int rows, int m, int kp, bool plain) {
  if (!pair && m == 1 && rows >= 4096 && kp >= 8192 && plain) return 4;
  return pair ? (m <= 4 ? 2 : 3) : (rows >= 4096 ? 1 : 0);
}
inline int class_rows(int c) { return (c == 0 || c == 4) ? 1 : (c == 3 ? 4 : 2); }
inline int class_waves(int c) { return c == 4 ? 16 : (c == 1 ? 8 : 4); }

template <int QT, int M>
void gemv_dispatch_class(int cls, int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  switch (cls) {
    case 0: gemv_dispatch_mode<QT, M, 1, 1, 4, false>(mode, grid, lds, st, a); break;
    case 1: gemv_dispatch_mode<QT, M, 2, 1, 8, false>(mode, grid, lds, st, a); break;
    case kGemvMfmaClass:  // 5..16 input rows on the matrix cores (block-quantized weights)
      if constexpr (M == 16 && QT != kF32) {
        if (a.res_add || a.amax_v || (a.xd && mode != kModeAdd) || (mode == kModeAdd && a.norm_w) ||
            (grid.y > 1 && mode != kModeAdd))
          throw HipError{"gemv: the matrix-core decode takes plain inputs, or accumulators in add mode"};
        switch (mode) {
          case kModeStore: qlaunch(gemv_mfma_kernel<QT, kModeStore>, grid, 256, 0, st, a); break;
          case kModeAdd:
            if (a.xd) qlaunch(gemv_mfma_kernel<QT, kModeAdd, true>, grid, 256, 0, st, a);
            else qlaunch(gemv_mfma_kernel<QT, kModeAdd>, grid, 256, 0, st, a);
            break;
          case kModePairSilu: qlaunch(gemv_mfma_kernel<QT, kModePairSilu>, grid, 256, 0, st, a); break;
          default: qlaunch(gemv_mfma_kernel<QT, kModePairGelu>, grid, 256, 0, st, a); break;
        }
      } else {
        throw HipError{"gemv: the matrix-core decode takes block-quantized weights and sixteen input rows"};
      }
      break;
    case 4:  // plain store / add only (see gemv_tile_class)
      if constexpr (M == 1) {
        if (a.res_add || a.xd || a.amax_v) throw HipError{"gemv: tile class 4 takes plain inputs only"};
        if (mode == kModeAdd) qlaunch(gemv_kernel<QT, 1, kModeAdd, 1, 1, 16, false>, grid, 1024, lds, st, a);
        else if (mode == kModeStore) qlaunch(gemv_kernel<QT, 1, kModeStore, 1, 1, 16, false>, grid, 1024, lds, st, a);
        else throw HipError{"gemv: tile class 4 takes the store and add epilogues"};
      } else {
        throw HipError{"gemv: tile class 4 takes one input row"};
      }
      break;
    case 2:
      if constexpr (M <= 4) gemv_dispatch_mode<QT, M, 2, 1, 4, true>(mode, grid, lds, st, a);
      else throw HipError{"gemv: tile class 2 takes at most four input rows"};
      break;
    default:
      if constexpr (M >= 8) gemv_dispatch_mode<QT, M, 4, 1, 4, true>(mode, grid, lds, st, a);
      else throw HipError{"gemv: tile class 3 takes eight or sixteen input rows"};
      break;
  }
}

// GEMV over M input rows (a power of two, at most 16) with tile class cls.
template <int QT>
void gemv_launch(int M, int cls, int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  switch (M) {
    case 1: gemv_dispatch_class<QT, 1>(cls, mode, grid, lds, st, a); break;
    case 2: gemv_dispatch_class<QT, 2>(cls, mode, grid, lds, st, a); break;
    case 4: gemv_dispatch_class<QT, 4>(cls, mode, grid, lds, st, a); break;
    case 8: gemv_dispatch_class<QT, 8>(cls, mode, grid, lds, st, a); break;
    default: gemv_dispatch_class<QT, 16>(cls, mode, grid, lds, st, a); break;
  }
}

// ------------------------------------------------------------ GEMM
template <int QT>
void gemm_dispatch(int mode, dim3 grid, hipStream_t st, const GemmArgs& a) {
  switch (mode) {
    case kModeStore: qlaunch(gemm_kernel<QT, kModeStore>, grid, 256, 0, st, a); break;
    case kModeAdd: qlaunch(gemm_kernel<QT, kModeAdd>, grid, 256, 0, st, a); break;
    case kModePairSilu: qlaunch(gemm_kernel<QT, kModePairSilu>, grid, 256, 0, st, a); break;
    default: qlaunch(gemm_kernel<QT, kModePairGelu>, grid, 256, 0, st, a); break;
  }
}

template <int QT, int NWV>
void gemm_ksplit_dispatch(int mode, dim3 grid, hipStream_t st, const GemmArgs& a) {
  const unsigned nt = 64 * NWV;
  switch (mode) {
    case kModeStore: qlaunch(gemm_ksplit_kernel<QT, kModeStore, NWV>, grid, nt, 0, st, a); break;
    case kModeAdd: qlaunch(gemm_ksplit_kernel<QT, kModeAdd, NWV>, grid, nt, 0, st, a); break;
    case kModePairSilu: qlaunch(gemm_ksplit_kernel<QT, kModePairSilu, NWV>, grid, nt, 0, st, a); break;
    default: qlaunch(gemm_ksplit_kernel<QT, kModePairGelu, NWV>, grid, nt, 0, st, a); break;
  }
}

template <int QT, int NT>
void gemm_bf16_dispatch(int mode, dim3 grid, hipStream_t st, const GemmArgs& a) {
  switch (mode) {
    case kModeStore: qlaunch(gemm_bf16_kernel<QT, kModeStore, NT>, grid, 256, 0, st, a); break;
    case kModeAdd: qlaunch(gemm_bf16_kernel<QT, kModeAdd, NT>, grid, 256, 0, st, a); break;
    case kModePairSilu: qlaunch(gemm_bf16_kernel<QT, kModePairSilu, NT>, grid, 256, 0, st, a); break;
    default: qlaunch(gemm_bf16_kernel<QT, kModePairGelu, NT>, grid, 256, 0, st, a); break;
  }
}

// Prefill GEMM kinds: the wide 64 x 128 f32 tile, the K-split 32 x 64 f32
// tile (four or eight waves), and the bf16 tile with one or three activation
// terms.
enum { kGemmWide = 0, kGemmKSplit = 1, kGemmBf16 = 2, kGemmBf16x3 = 3, kGemmKSplit8 = 4 };

template <int QT>
void gemm_launch(int kind, int mode, dim3 grid, hipStream_t st, const GemmArgs& a) {
  if (kind == kGemmKSplit) {
    gemm_ksplit_dispatch<QT, 4>(mode, grid, st, a);
  } else if (kind == kGemmKSplit8) {
    gemm_ksplit_dispatch<QT, 8>(mode, grid, st, a);
  } else if (kind == kGemmWide) {
    gemm_dispatch<QT>(mode, grid, st, a);
  } else {
    if constexpr (QT == kQ8_0 || QT == kQ4_0) {
      if (kind == kGemmBf16x3) gemm_bf16_dispatch<QT, 3>(mode, grid, st, a);
      else gemm_bf16_dispatch<QT, 1>(mode, grid, st, a);
    } else {
      throw HipError{"gemm: no bf16 tile for this weight type"};
    }
  }
}

#define QD_KERNEL_TYPES(X) X(kF32) X(kQ4_0) X(kQ8_0) X(kQ4_K) X(kQ6_K)
#define QD_EXTERN(T)                                                                                \
  extern template void gemv_launch<T>(int, int, int, dim3, size_t, hipStream_t, const GemvArgs&); \
  extern template void gemm_launch<T>(int, int, dim3, hipStream_t, const GemmArgs&);
QD_KERNEL_TYPES(QD_EXTERN)
#undef QD_EXTERN

}  // namespace qd
