// Dispatch of the persistent streaming GEMV kernels (gemv_stream.hpp) to the
// per-row-count translation units gemv_stream_m<M>.hip.
#include "gemv_stream.hpp"

namespace nvfp4 {

hipError_t launch_gemv_stream(const GemvPlan& p, int M, int64_t N, int64_t K, const uint8_t* xc,
                              const uint8_t* xs, const float* xg, const uint8_t* wc,
                              const uint8_t* ws, const float* wg, void* y, int out_bf16,
                              void* workspace, hipStream_t s, const uint16_t* xb, int64_t ldx,
                              uint8_t* oc, uint8_t* os, float* og, int rms, float eps,
                              float* ho, const float* sgs, const float* xf,
                              const uint32_t* amax_in, int qslice, uint32_t* amax_out,
                              int64_t ldh, uint16_t* gu) {
  GemvArgs a = {};
  a.sgs = sgs;
  a.xf = xf;
  a.amax_in = amax_in;
  a.qslice = qslice;
  a.amax_out = amax_out;
  a.ldh = ldh;
  a.gu = gu;
  a.rms = rms;
  a.eps = eps;
  a.ho = ho;
  a.xb = xb;
  a.ldx = ldx;
  a.oc = oc;
  a.os = os;
  a.og = og;
  a.xc = xc;
  a.xs = xs;
  a.xg = xg;
  a.wc = wc;
  a.ws = ws;
  a.wg = wg;
  a.y = y;
  a.N = (int)N;
  a.n_pad = p.tiles * kTileN;
  a.K = (int)K;
  a.kc = p.kc;
  a.kg = p.kc / 4;
  a.cpw = p.cpw;
  a.cps = p.cps;
  a.splits = p.splits;
  a.batch = p.batch;
  a.waves = p.waves;
  a.part = p.splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                   kCounterBytes)
                        : nullptr;
  a.cnt = static_cast<uint32_t*>(workspace);
  a.out_bf16 = out_bf16;
  a.nontemporal = p.nontemporal;
  a.tiles = p.tiles;
  const bool mf = p.kind == kGemvMfma;
  if (!mf && M > 3) return hipErrorInvalidValue;          // the VALU dot: M <= 3
  switch (M) {
    case 1: return launch_stream_rows<1>(p, a, s, mf);
    case 2: return launch_stream_rows<2>(p, a, s, mf);
    case 3: return launch_stream_rows<3>(p, a, s, mf);
    case 4: return launch_stream_rows<4>(p, a, s, mf);
    case 5: return launch_stream_rows<5>(p, a, s, mf);
    case 6: return launch_stream_rows<6>(p, a, s, mf);
    case 7: return launch_stream_rows<7>(p, a, s, mf);
    case 8: return launch_stream_rows<8>(p, a, s, mf);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4
