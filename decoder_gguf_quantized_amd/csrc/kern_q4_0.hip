// GEMV and GEMM instantiations for Q4_0 weights (compiled on their own,
// in parallel with the other weight types).
#include "dispatch.hpp"

namespace qd {
template void gemv_launch<kQ4_0>(int, int, int, dim3, size_t, hipStream_t, const GemvArgs&);
template void gemm_launch<kQ4_0>(int, int, dim3, hipStream_t, const GemmArgs&);
}  // namespace qd
