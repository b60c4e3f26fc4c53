// prefill_channel.hip -- chunked prefill with one decay per key channel (KDA form).
#include "common.h"
#include "internal.h"

namespace lt2 {

size_t prefill_channel_ws_bytes(int, int, int, int, int) { return 0; }

hipError_t launch_prefill_channel(const GdnArgs &, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace lt2
