// Decode kernel instances for io dtype bf16 with KV dtype fp8 (all head_dim / group
// combinations, block sizes 64 .. 512), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_bf16_fp8_large(const LaunchSpec& ls) { return launch_decode<kBF16, kFP8, true>(ls); }
}  // namespace pa
