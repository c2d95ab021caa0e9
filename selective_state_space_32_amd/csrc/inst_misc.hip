// Explicit instantiations of libssmscan's launch templates (see launch.h); the library's
// translation units are compiled in parallel and linked together.
#include "launch.h"

namespace ssmlib {
template int launch_step<1, float>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<2, float>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<4, float>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<8, float>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<16, float>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<1, uint16_t>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<2, uint16_t>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<4, uint16_t>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<8, uint16_t>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);
template int launch_step<16, uint16_t>(float *, const void *, const void *, const float *, const void *, const void *, const float *, const void *, void *, const ssm_dims *, hipStream_t, const float *, int, int);

template int launch_conv<float>(int, bool, const void *, const float *, const float *, const void *, void *, void *,
                                const ssm_dims *, hipStream_t);
template int launch_conv<uint16_t>(int, bool, const void *, const float *, const float *, const void *, void *,
                                   void *, const ssm_dims *, hipStream_t);
template void launch_conv_bwd<float>(int, bool, const void *, const float *, const float *, const void *,
                                     const void *, void *, float *, float *, void *, const ssm_dims *, hipStream_t);
template void launch_conv_bwd<uint16_t>(int, bool, const void *, const float *, const float *, const void *,
                                        const void *, void *, float *, float *, void *, const ssm_dims *, hipStream_t);

void launch_ssd(const void *x, const void *dt, const float *A, const void *B, const void *C, const float *D,
                const void *z, const float *dt_bias, int softplus, void *y, float *last_state, int64_t bsz,
                int64_t L, int64_t H, int64_t G, hipStream_t st, const float *h0, int64_t P, int64_t N, bool f32) {
    const int64_t vh = P > 64 ? P / 64 : 1;   // 64-channel virtual heads per head
    const dim3 grid((unsigned)(bsz * H * vh)), block(ssm::kSsdThreads);
    if (f32) {   // fp32 I/O: dstate 32 or 64
        auto kern = (P < 64 || N < 64) ? ssm::ssd_chunk_kernel<true, 64, true> : ssm::ssd_chunk_kernel<false, 64, true>;
        hipLaunchKernelGGL(kern, grid, block, 0, st, static_cast<const float *>(x), static_cast<const float *>(dt), A,
                           static_cast<const float *>(B), static_cast<const float *>(C), D,
                           static_cast<const float *>(z), dt_bias, static_cast<float *>(y), last_state, L, (int)H,
                           (int)G, softplus, h0, (int)P, (int)N);
        return;
    }
    auto kern = N == 128 ? ssm::ssd_chunk_kernel<false, 128>
                         : (P < 64 || N < 64) ? ssm::ssd_chunk_kernel<true> : ssm::ssd_chunk_kernel<false>;
    hipLaunchKernelGGL(kern, grid, block, 0, st, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dt),
                       A, static_cast<const uint16_t *>(B), static_cast<const uint16_t *>(C), D,
                       static_cast<const uint16_t *>(z), dt_bias, static_cast<uint16_t *>(y), last_state, L, (int)H,
                       (int)G, softplus, h0, (int)P, (int)N);
}

}  // namespace ssmlib
