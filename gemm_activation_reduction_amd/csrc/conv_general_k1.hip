// Instantiations of the general-geometry convolution for 1x1 kernels (see
// conv_general_kernel.h).
#include "conv_general_kernel.h"

namespace fconv {

hipError_t launch_geo_k1(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                         hipStream_t stream) {
    if (p.KS != 1 || (p.stride != 1 && p.stride != 2)) return hipErrorInvalidValue;
    const bool s1 = p.stride == 1;
    if (p.BN == 128 && p.bf16)
        return s1 ? launch_geo_act<true, GeoTile<1, 1, 2>>(p, x, wpk, b, dst, stream)
                  : launch_geo_act<true, GeoTile<1, 2, 2>>(p, x, wpk, b, dst, stream);
    // fp32 1x1 stride 1 with 16-byte halo runs: LDS-DMA staging
    if (!p.bf16 && s1 && p.pad == 0 && p.W % 4 == 0 && (uintptr_t)x % 16 == 0) {
        if (p.BN == 128) return launch_geo_act<false, GeoTile<1, 1, 2, 4>, 1>(p, x, wpk, b, dst, stream);
        if (p.BN == 16) return launch_geo_act<false, GeoTile<1, 1, 1, 2, 16>, 1>(p, x, wpk, b, dst, stream);
        if (p.BN == 32) return launch_geo_act<false, GeoTile<1, 1, 1, 2, 32>, 1>(p, x, wpk, b, dst, stream);
        if (p.BN == 64) return launch_geo_act<false, GeoTile<1, 1>, 1>(p, x, wpk, b, dst, stream);
    }
    if (p.BN == 128)
        return s1 ? launch_geo_act<false, GeoTile<1, 1, 2>>(p, x, wpk, b, dst, stream)
                  : launch_geo_act<false, GeoTile<1, 2, 2>>(p, x, wpk, b, dst, stream);
    if (p.BN == 16)
        return s1 ? launch_geo_dtype<GeoTile<1, 1, 1, 2, 16>>(p, x, wpk, b, dst, stream)
                  : launch_geo_dtype<GeoTile<1, 2, 1, 2, 16>>(p, x, wpk, b, dst, stream);
    if (p.BN == 32)
        return s1 ? launch_geo_dtype<GeoTile<1, 1, 1, 2, 32>>(p, x, wpk, b, dst, stream)
                  : launch_geo_dtype<GeoTile<1, 2, 1, 2, 32>>(p, x, wpk, b, dst, stream);
    if (p.BN == 64)
        return s1 ? launch_geo_dtype<GeoTile<1, 1>>(p, x, wpk, b, dst, stream)
                  : launch_geo_dtype<GeoTile<1, 2>>(p, x, wpk, b, dst, stream);
    return hipErrorInvalidValue;
}

}  // namespace fconv
