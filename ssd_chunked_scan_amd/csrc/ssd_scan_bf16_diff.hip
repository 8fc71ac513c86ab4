// The bf16 head kernel with the diff segsum on its output path (segsum
// ablation, page "GPU Hierarchy Meets Structured Matrices", abstract), chunk
// 256, dstate 64 or 128, headdim blocks of 32 or 64; full pass only (the
// split-local pass is the same for every segsum: the hierarchy kernels).
#include "ssd_scan_bf16.hpp"

namespace ssd {

#define SSD_SCAN_CASE(n, pb)                                                            \
    if (N == n && PB == pb) {                                                            \
        return launch_scan_bf16<256, n, pb, kSegsumDiff>(a, stream);                    \
    }

bool launch_scan_bf16_diff(int N, int PB, const ChunkArgs &a, hipStream_t stream) {
    SSD_SCAN_CASE(64, 32)
    SSD_SCAN_CASE(64, 64)
    SSD_SCAN_CASE(128, 32)
    SSD_SCAN_CASE(128, 64)
    return false;
}

}  // namespace ssd
