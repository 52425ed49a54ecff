// placeholder until the channel-gated bf16 kernel lands
#include "launch.h"
namespace gdr {
hipError_t launch_gdr2_bf16(const ChunkArgs&) { return hipErrorNotSupported; }
}
