// Decode kernel instances for io dtype f32 with KV dtype f32 (all head_dim / group
// combinations, block sizes 8 .. 32), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_f32_f32(const LaunchSpec& ls) { return launch_decode<kF32, kF32, false>(ls); }
}  // namespace pa
