// Decode kernel instances for io dtype f16 with KV dtype fp8 (all head_dim / group
// combinations, block sizes 8 .. 32), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_f16_fp8(const LaunchSpec& ls) { return launch_decode<kF16, kFP8, false>(ls); }
}  // namespace pa
