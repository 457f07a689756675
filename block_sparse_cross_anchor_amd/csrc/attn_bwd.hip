// placeholder until the bf16 backward lands
#include "internal.h"
namespace sxa {
hipError_t launch_bwd_bf16(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
}
