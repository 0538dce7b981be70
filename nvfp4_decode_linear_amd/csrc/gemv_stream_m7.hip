// Streaming GEMV kernels for M = 7 activation rows (see gemv_stream.hpp).
#include "gemv_stream.hpp"

namespace nvfp4 {

template <>
hipError_t launch_stream_rows<7>(const GemvPlan& p, const GemvArgs& a, hipStream_t s, bool mf) {
  return mf ? launch_m<7, true>(p, a, s) : hipErrorInvalidValue;
}

}  // namespace nvfp4
