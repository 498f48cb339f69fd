// Sparse MLA decode attention over resolved slots (placeholder until the MFMA kernel lands).
#include "hs_internal.h"

namespace hs {

int attend_splits(const Geometry& g) { (void)g; return 1; }
size_t attend_partial_floats(const Geometry& g) { (void)g; return 0; }

hipError_t launch_attend(const Geometry& g, const LayerTables& t, int32_t n_req, const void* q, const int32_t* slots,
                         float scale, void* out, float* lse, hipStream_t s) {
  (void)g; (void)t; (void)n_req; (void)q; (void)slots; (void)scale; (void)out; (void)lse; (void)s;
  return hipErrorNotSupported;
}

}  // namespace hs
