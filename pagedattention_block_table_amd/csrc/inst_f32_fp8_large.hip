// Decode kernel instances for io dtype f32 with KV dtype fp8 (all head_dim / group
// combinations, block sizes 64 .. 512), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_f32_fp8_large(const LaunchSpec& ls) { return launch_decode<kF32, kFP8, true>(ls); }
}  // namespace pa
