#include "gdn_device.h"
#include "gdn_internal.h"
namespace gdn {
int launch_chunk(const Problem&, void*, bool, void*) { return int(hipErrorNotSupported); }
}
