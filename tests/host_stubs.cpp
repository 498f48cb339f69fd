// Host-only stand-ins for the device-side functions of libhs, so that the host API
// (hs_api.cpp: configuration checks, memory plans, argument validation, handle lifetime) can
// be built with a plain host compiler and run under AddressSanitizer / UBSan on a machine
// without a GPU (tests/test_sanitizers.py).  Every launch reports hipErrorNotSupported; the
// size helpers return plain bounds of the right order.  Not part of the library.
#include "hs_internal.h"

namespace hs {

void prepare_resolve() {}
void prepare_append() {}
void prepare_topk() {}
void prepare_attend() {}

size_t resolve_lds_bytes(int64_t cap, int32_t k, int32_t B) {  // the order of the resolver's LDS plan
  const size_t W = (size_t)((cap + 31) >> 5), HB = (size_t)((B + 31) >> 5);
  return (3 * HB + W + 3 * (size_t)k + 16 + (W + 1) / 2) * 4;
}

int attend_splits(const Geometry& g, int n_req) {
  const int s = 256 / (n_req > 0 ? n_req : 1);
  return s < 1 ? 1 : (s > 16 ? 16 : s);
}

size_t attend_partial_floats(const Geometry& g) { return (size_t)17 * (2 * 16 + 16 * 512); }

int64_t attend_noalloc_partials(const Geometry& g, int32_t n_req, int32_t heads) {
  const int s = attend_splits(g, n_req);
  return s > 1 ? (int64_t)n_req * s : 0;
}

hipError_t prepare_attend_noalloc(int) { return hipErrorNotSupported; }

hipError_t launch_resolve(const Geometry&, const LayerTables&, int32_t, const uint8_t*, int32_t, const int32_t*,
                          int32_t*, int32_t*, int32_t*, bool, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fetch(const Geometry&, const LayerTables&, const uint8_t*, int32_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_reset(const Geometry&, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, uint32_t*, int32_t, int32_t,
                        hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_append(const Geometry&, const LayerTables&, uint8_t*, int32_t, const int32_t*, const void*, int64_t,
                         int32_t*, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_append_pages(const Geometry&, const LayerTables&, uint8_t*, int32_t, const int32_t*, const void*,
                               int64_t, int32_t*, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_offload(const void*, int64_t, uint8_t*, int64_t, int64_t, uint8_t*, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_topk(const Geometry&, int32_t, const float*, int64_t, const int32_t*, int32_t*, int32_t*,
                       int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_stream_read(const void*, size_t, uint32_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attend(const Geometry&, const LayerTables&, int32_t, const void*, const int32_t*, const int32_t*,
                         const int32_t*, float, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_attend_noalloc(const Geometry&, const LayerTables&, int, int32_t, int32_t, const void*,
                                 const int32_t*, float, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_attend_part(const Geometry&, const LayerTables&, int32_t, bool, const void*, const int32_t*,
                              const int32_t*, const int32_t*, float, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace hs
