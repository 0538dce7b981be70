// Streaming GEMV kernels for M = 3 activation rows (see gemv_stream.hpp).
#include "gemv_stream.hpp"

namespace nvfp4 {

template <>
hipError_t launch_stream_rows<3>(const GemvPlan& p, const GemvArgs& a, hipStream_t s, bool mf) {
  return mf ? launch_m<3, true>(p, a, s) : launch_m<3, false>(p, a, s);
}

}  // namespace nvfp4
