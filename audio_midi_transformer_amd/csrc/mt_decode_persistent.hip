// Persistent single-launch decode step (placeholder until implemented).
#include <hip/hip_runtime.h>
#include "mt_internal.h"
namespace mt {
bool persistent_supported(int, int, int, int, int) { return false; }
size_t persistent_xbuf_bytes(int, int, int, int, int, int) { return 0; }
hipError_t launch_persistent_decode(const PersistentArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mt
