// Chunked WKV-7 prefill (placeholder until the MFMA kernel lands).
#include "wkv7_internal.hpp"

namespace rwkv7 {
hipError_t launch_chunked(const WkvCall&) { return hipErrorNotSupported; }
}  // namespace rwkv7
