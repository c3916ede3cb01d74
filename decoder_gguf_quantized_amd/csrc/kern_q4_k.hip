// GEMV and GEMM instantiations for Q4_K weights (compiled on their own,
// in parallel with the other weight types).
#include "dispatch.hpp"

namespace qd {
template void gemv_launch<kQ4_K>(int, int, int, dim3, size_t, hipStream_t, const GemvArgs&);
template void gemm_launch<kQ4_K>(int, int, dim3, hipStream_t, const GemmArgs&);
}  // namespace qd
