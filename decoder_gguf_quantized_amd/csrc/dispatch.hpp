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
template <int QT, int M, int R, int U, int NW = 4>
void gemv_dispatch_mode(int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  const unsigned nt = 64 * NW;
  if (a.amax_v) {  // the LM head of one row with the greedy choice in its epilogue
    if constexpr (M == 1) {
      if (mode != kModeStore || a.xd) throw HipError{"gemv: the fused argmax needs the plain store epilogue"};
      if (a.res_add) qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, true, false, true>, grid, nt, lds, st, a);
      else qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, false, false, true>, grid, nt, lds, st, a);
      return;
    } else {
      throw HipError{"gemv: the fused argmax takes one input row"};
    }
  }
  if (a.res_add) {  // residual prologue (sandwich norms): store and pair modes
    switch (mode) {
      case kModeStore: qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, true>, grid, nt, lds, st, a); break;
      case kModePairSilu: qlaunch(gemv_kernel<QT, M, kModePairSilu, R, U, NW, true>, grid, nt, lds, st, a); break;
      case kModePairGelu: qlaunch(gemv_kernel<QT, M, kModePairGelu, R, U, NW, true>, grid, nt, lds, st, a); break;
      default: throw HipError{"gemv: residual prologue with an add epilogue"};
    }
    return;
  }
  if (a.xd) {  // input from decode attention's accumulators: the O projection (store or add)
    switch (mode) {
      case kModeStore: qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, false, true>, grid, nt, lds, st, a); break;
      case kModeAdd: qlaunch(gemv_kernel<QT, M, kModeAdd, R, U, NW, false, true>, grid, nt, lds, st, a); break;
      default: throw HipError{"gemv: attention-accumulator input with a pair epilogue"};
    }
    return;
  }
  switch (mode) {
    case kModeStore: qlaunch(gemv_kernel<QT, M, kModeStore, R, U, NW, false>, grid, nt, lds, st, a); break;
    case kModeAdd: qlaunch(gemv_kernel<QT, M, kModeAdd, R, U, NW, false>, grid, nt, lds, st, a); break;
    case kModePairSilu: qlaunch(gemv_kernel<QT, M, kModePairSilu, R, U, NW, false>, grid, nt, lds, st, a); break;
    default: qlaunch(gemv_kernel<QT, M, kModePairGelu, R, U, NW, false>, grid, nt, lds, st, a); break;
  }
}

// (R rows per wave, U units per lane per row, NW waves per workgroup):
//   0: R = 4, U = 1 for rows of at most 64 units (one unit per lane);
//   1: R = 2, U = 2 for rows of 65..128 units;
//   2: R = 2, U = 4 for longer rows;
//   3: as 2 with eight-wave workgroups, for long rows with many row groups:
//      the input row is staged once per CU instead of twice (same LDS).
// LDS budget of the GEMV's staged input rows (the CU has 160 KB; the rest is
// left for the kernel's own small arrays).
constexpr size_t kGemvLdsMax = 128 * 1024;

// Largest input-row count M (a power of two, at most 16) whose staged rows fit
// the LDS budget for the shortest row of each tile class (class 0: any row;
// class 1: 65 units; classes 2 and 3: 129 units; Q8_0 / Q6_K 16 weights per
// unit, Q4_0 / Q4_K 32, F32 4); combinations beyond it cannot be requested and
// are not instantiated.
constexpr int gemv_max_m(int qt, int ru) {
  if (ru == 0) return 16;
  const size_t units = ru == 1 ? 65 : 129;
  const size_t k = units * (int8_layout(qt) ? 16 : (nibble_layout(qt) ? 32 : 4));
  const size_t per_row = k * 4 + (nibble_layout(qt) ? k / 32 * 4 : 0);
  int m = 16;
  while (m > 1 && per_row * m > kGemvLdsMax) m /= 2;
  return m;
}

template <int QT, int M, int RU, int R, int U, int NW = 4>
void gemv_dispatch_fit(int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  if constexpr (M <= gemv_max_m(QT, RU)) gemv_dispatch_mode<QT, M, R, U, NW>(mode, grid, lds, st, a);
  else throw HipError{"gemv: input rows exceed the LDS budget of the tile class"};
}

template <int QT, int M>
void gemv_dispatch_ru(int ru, int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  switch (ru) {
    case 0: gemv_dispatch_fit<QT, M, 0, 4, 1>(mode, grid, lds, st, a); break;
    case 1: gemv_dispatch_fit<QT, M, 1, 2, 2>(mode, grid, lds, st, a); break;
    case 3: gemv_dispatch_fit<QT, M, 3, 2, 4, 8>(mode, grid, lds, st, a); break;
    default: gemv_dispatch_fit<QT, M, 2, 2, 4>(mode, grid, lds, st, a); break;
  }
}

// tile classes: 0 = four rows x one unit per lane, 1 = two rows x two units,
// 2 = two rows x four units, 3 = class 2 in eight-wave workgroups
inline int ru_rows(int ru) { return ru == 0 ? 4 : 2; }
inline int ru_waves(int ru) { return ru == 3 ? 8 : 4; }

template <int QT>
void gemv_dispatch_m(int M, int ru, int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  switch (M) {
    case 1: gemv_dispatch_ru<QT, 1>(ru, mode, grid, lds, st, a); break;
    case 2: gemv_dispatch_ru<QT, 2>(ru, mode, grid, lds, st, a); break;
    case 4: gemv_dispatch_ru<QT, 4>(ru, mode, grid, lds, st, a); break;
    case 8: gemv_dispatch_ru<QT, 8>(ru, mode, grid, lds, st, a); break;
    default: gemv_dispatch_ru<QT, 16>(ru, mode, grid, lds, st, a); break;
  }
}

// GEMV over M input rows with tile class ru (see gemv_dispatch_ru).
template <int QT>
void gemv_launch(int M, int ru, int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  gemv_dispatch_m<QT>(M, ru, mode, grid, lds, st, a);
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
