// Decode kernel instances for io dtype f16 with KV dtype f16 (all head_dim / group
// combinations, block sizes 8 .. 32), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_f16_f16(const LaunchSpec& ls) { return launch_decode<kF16, kF16, false>(ls); }
}  // namespace pa
