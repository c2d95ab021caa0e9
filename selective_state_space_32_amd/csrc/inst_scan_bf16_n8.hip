// Explicit instantiations of libssmscan's launch templates (see launch.h); the library's
// translation units are compiled in parallel and linked together.
#include "launch.h"

namespace ssmlib {
template int launch_scan<8, uint16_t>(const void *, const void *, const float *, const void *, const void *, const float *, const void *, const float *, int, const float *, void *, float *, const ssm_dims *, const Plan &, void *, hipStream_t, const ConvArgs *, float *, const int32_t *);

}  // namespace ssmlib
