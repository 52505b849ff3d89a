// read_probe.hpp -- host launcher of the read-bandwidth reference kernel
// (read_probe.hip), internal to libresident_topk.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rt {

// Reads the n16 16-byte words at p once (a contiguous chunk per wave, one
// 4-wave workgroup per CU, non-temporal loads, eight in flight per lane, no
// other work); sink must hold num_cus * 4 words.
hipError_t launch_read_probe(const void *p, int64_t n16, uint32_t *sink, int num_cus, hipStream_t stream);

}  // namespace rt
