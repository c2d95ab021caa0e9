// Explicit instantiations of libssmscan's launch templates (see launch.h); the library's
// translation units are compiled in parallel and linked together.
#include "launch.h"

namespace ssmlib {
template int launch_bwd<1, float>(const BwdArgs &, const ssm_dims *, const Plan &, size_t, void *, hipStream_t);
template int launch_bwd<2, float>(const BwdArgs &, const ssm_dims *, const Plan &, size_t, void *, hipStream_t);
template int launch_bwd<4, float>(const BwdArgs &, const ssm_dims *, const Plan &, size_t, void *, hipStream_t);
template int launch_bwd<8, float>(const BwdArgs &, const ssm_dims *, const Plan &, size_t, void *, hipStream_t);
template int launch_bwd<16, float>(const BwdArgs &, const ssm_dims *, const Plan &, size_t, void *, hipStream_t);

}  // namespace ssmlib
