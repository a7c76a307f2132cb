// Decode kernel instances for io dtype bf16 with KV dtype bf16 (all head_dim / group
// combinations, block sizes 64 .. 512), compiled as a translation unit of their own.
#include "pa_decode_impl.h"

namespace pa {
int launch_bf16_bf16_large(const LaunchSpec& ls) { return launch_decode<kBF16, kBF16, true>(ls); }
}  // namespace pa
