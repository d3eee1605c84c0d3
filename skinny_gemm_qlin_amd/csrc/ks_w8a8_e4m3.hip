// ks_w8a8_e4m3.hip -- the K-slice decode kernels for FP8 W8A8 with E4M3 activation codes (ks_kernels.hpp), planned in
// gemv.hip.
#include "ks_launch.hpp"

namespace qlin {

hipError_t launch_ks_w8a8_e4m3(const KsArgs& a, const KsPlan& p, int w_fmt, hipStream_t st) {
    return w_fmt == kFmtE5M2 ? run_ks<kKsW8A8, kFmtE4M3, kFmtE5M2>(a, p, st) : run_ks<kKsW8A8, kFmtE4M3, kFmtE4M3>(a, p, st);
}

}  // namespace qlin
