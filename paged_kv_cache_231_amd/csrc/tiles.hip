// Chunked-prefill tile kernel (MFMA).  Not built yet: every query is served
// by the per-query kernels until this kernel lands.

#include "device_common.h"

namespace pkv {

bool tiles_supported(const TileArgs &, pkv_dtype) { return false; }

hipError_t launch_tiles(const TileArgs &, pkv_dtype, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
