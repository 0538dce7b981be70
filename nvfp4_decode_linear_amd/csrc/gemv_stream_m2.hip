// Streaming GEMV kernels for M = 2 activation rows (see gemv_stream.hpp).
#include "gemv_stream.hpp"

namespace nvfp4 {

template <>
hipError_t launch_stream_rows<2>(const GemvPlan& p, const GemvArgs& a, hipStream_t s, bool mf) {
  return mf ? launch_m<2, true>(p, a, s) : launch_m<2, false>(p, a, s);
}

}  // namespace nvfp4
