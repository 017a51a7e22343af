// Grouped int8-MFMA expert FFN (many tokens per expert).
#include "internal.h"

namespace maple {

hipError_t launch_grouped_ffn(const Dims&, int64_t, const void*, bool, const uint8_t*,
                              const float*, const Workspace&, float*, const float*, float*,
                              hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace maple
