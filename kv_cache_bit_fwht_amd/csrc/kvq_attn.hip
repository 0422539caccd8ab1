// placeholder: attention kernels (replaced below)
#include "kvq_internal.hpp"
namespace kvq {
size_t decode_ws_bytes(const kvq_shape&, int, int) { return 0; }
size_t error_ws_bytes(const kvq_shape&, int, int) { return 0; }
hipError_t launch_decode_generic(const AttnProblem&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_error(const AttnProblem&, hipStream_t) { return hipErrorNotSupported; }
bool fast_decode_supported(const kvq_packed&, const kvq_packed&, int) { return false; }
hipError_t launch_decode_fast(const AttnProblem&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_rfft_quantize(const uint16_t*, const kvq_packed&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_rfft_dequant(const kvq_packed&, float*, hipStream_t) { return hipErrorNotSupported; }
}
