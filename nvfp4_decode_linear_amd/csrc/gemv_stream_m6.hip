// Streaming GEMV kernels for M = 6 activation rows (see gemv_stream.hpp).
#include "gemv_stream.hpp"

namespace nvfp4 {

template <>
hipError_t launch_stream_rows<6>(const GemvPlan& p, const GemvArgs& a, hipStream_t s, bool mf) {
  return mf ? launch_m<6, true>(p, a, s) : hipErrorInvalidValue;
}

}  // namespace nvfp4
