// Instantiations of the bf16 head kernel for chunk size 128.
#include "ssd_scan_bf16.hpp"

namespace ssd {

#define SSD_SCAN_CASE(q, n, pb)                                                         \
    if (N == n && PB == pb) {                                                            \
        launch_scan_bf16<q, n, pb>(a, stream);                                          \
        return true;                                                                    \
    }

bool launch_scan_bf16_q128(int N, int PB, const ChunkArgs &a, hipStream_t stream) {
    SSD_SCAN_CASE(128, 16, 16)
    SSD_SCAN_CASE(128, 16, 32)
    SSD_SCAN_CASE(128, 16, 64)
    SSD_SCAN_CASE(128, 16, 128)
    SSD_SCAN_CASE(128, 32, 16)
    SSD_SCAN_CASE(128, 32, 32)
    SSD_SCAN_CASE(128, 32, 64)
    SSD_SCAN_CASE(128, 32, 128)
    SSD_SCAN_CASE(128, 64, 16)
    SSD_SCAN_CASE(128, 64, 32)
    SSD_SCAN_CASE(128, 64, 64)
    SSD_SCAN_CASE(128, 64, 128)
    SSD_SCAN_CASE(128, 128, 16)
    SSD_SCAN_CASE(128, 128, 32)
    SSD_SCAN_CASE(128, 128, 64)
    return false;
}

}  // namespace ssd
