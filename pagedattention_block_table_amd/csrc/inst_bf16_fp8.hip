// Decode kernel instances for io dtype bf16 with KV dtype fp8 (all head_dim / group
// combinations, block sizes 8 .. 32), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_bf16_fp8(const LaunchSpec& ls) { return launch_decode<kBF16, kFP8, false>(ls); }
}  // namespace pa
