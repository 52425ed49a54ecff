// placeholder: bf16 MFMA kernels are added next
#include "gdr_device.h"
#include "launch.h"
namespace gdr {
hipError_t launch_chunk_bf16(const ChunkArgs&) { return hipErrorNotSupported; }
hipError_t launch_gdr2_bf16(const ChunkArgs&) { return hipErrorNotSupported; }
}
