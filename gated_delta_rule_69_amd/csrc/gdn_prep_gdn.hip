// Chunk preparation kernels of the GDN variant (one translation unit per variant keeps
// the per-variant kernels compiling in parallel).
#include "gdn_chunk.h"

namespace gdn {

int launch_prep_gdn(const Problem& p, void* ws, bool want_out, void* stream) {
  return launch_prep_variant<GDN_VARIANT_GDN>(p, ws, want_out, stream);
}

}  // namespace gdn
