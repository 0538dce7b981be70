// Streaming GEMV kernels for M = 1 activation row (see gemv_stream.hpp).
#include "gemv_stream.hpp"

namespace nvfp4 {

template <>
hipError_t launch_stream_rows<1>(const GemvPlan& p, const GemvArgs& a, hipStream_t s, bool mf) {
  return mf ? launch_m<1, true>(p, a, s) : launch_m<1, false>(p, a, s);
}

}  // namespace nvfp4
