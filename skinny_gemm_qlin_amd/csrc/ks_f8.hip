// ks_f8.hip -- the K-slice decode kernels for E4M3 weight-only (ks_kernels.hpp), planned in
// gemv.hip.
#include "ks_launch.hpp"

namespace qlin {

hipError_t launch_ks_f8(const KsArgs& a, const KsPlan& p, hipStream_t st) { return run_ks<kKsF8>(a, p, st); }

}  // namespace qlin
