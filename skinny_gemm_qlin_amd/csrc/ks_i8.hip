// ks_i8.hip -- the K-slice decode kernels for W8A8 INT8 (ks_kernels.hpp), planned in
// gemv.hip.
#include "ks_launch.hpp"

namespace qlin {

hipError_t launch_ks_i8(const KsArgs& a, const KsPlan& p, hipStream_t st) { return run_ks<kKsI8>(a, p, st); }

}  // namespace qlin
