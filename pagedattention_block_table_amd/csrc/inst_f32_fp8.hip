// Decode kernel instances for io dtype f32 with KV dtype fp8 (all head_dim / group
// combinations, block sizes 8 .. 32), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_f32_fp8(const LaunchSpec& ls) { return launch_decode<kF32, kFP8, false>(ls); }
}  // namespace pa
