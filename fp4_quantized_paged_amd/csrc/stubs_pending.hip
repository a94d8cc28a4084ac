// Entry points whose kernels are not built yet: they report "not supported".
#include "kvq_launch.h"

namespace kvq {
hipError_t launch_store_nvfp4(const StoreNvfp4Launch &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_mla(const DecodeMlaLaunch &, const MlaPlan &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kvq
