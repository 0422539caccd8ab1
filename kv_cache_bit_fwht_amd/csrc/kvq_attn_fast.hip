// MFMA decode-attention kernel (filled in below).
#include "kvq_internal.hpp"
namespace kvq {
bool fast_decode_supported(const kvq_packed&, const kvq_packed&, int) { return false; }
hipError_t launch_decode_fast(const AttnProblem&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kvq
