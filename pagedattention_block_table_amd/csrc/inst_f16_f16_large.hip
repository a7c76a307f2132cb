// Decode kernel instances for io dtype f16 with KV dtype f16 (all head_dim / group
// combinations, block sizes 64 .. 512), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_f16_f16_large(const LaunchSpec& ls) { return launch_decode<kF16, kF16, true>(ls); }
}  // namespace pa
