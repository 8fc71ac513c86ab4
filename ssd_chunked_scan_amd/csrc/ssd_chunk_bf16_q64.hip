// Instantiations of the bf16 chunk kernel for chunk size 64.
#include "ssd_chunk_bf16.hpp"

namespace ssd {

#define SSD_BF16_CASE(q, n, pb)                                                         \
    if (N == n && PB == pb) {                                                            \
        hipLaunchKernelGGL((ssd_chunk_bf16_kernel<q, n, pb>), grid,                     \
                           dim3(Bf16Cfg<q, n, pb>::THREADS), 0, stream, a);              \
        return true;                                                                    \
    }

bool launch_chunk_bf16_q64(int N, int PB, const ChunkArgs &a, hipStream_t stream) {
    const dim3 grid(a.units);
    SSD_BF16_CASE(64, 16, 16)
    SSD_BF16_CASE(64, 16, 32)
    SSD_BF16_CASE(64, 16, 64)
    SSD_BF16_CASE(64, 16, 128)
    SSD_BF16_CASE(64, 32, 16)
    SSD_BF16_CASE(64, 32, 32)
    SSD_BF16_CASE(64, 32, 64)
    SSD_BF16_CASE(64, 32, 128)
    SSD_BF16_CASE(64, 64, 16)
    SSD_BF16_CASE(64, 64, 32)
    SSD_BF16_CASE(64, 64, 64)
    SSD_BF16_CASE(64, 64, 128)
    SSD_BF16_CASE(64, 128, 16)
    SSD_BF16_CASE(64, 128, 32)
    SSD_BF16_CASE(64, 128, 64)
    SSD_BF16_CASE(64, 128, 128)
    return false;
}

}  // namespace ssd
