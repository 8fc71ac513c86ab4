// Per-group operands of the bf16 forward pass, computed once per (batch row,
// group, chunk) and shared by every head of the group.
//
// Page "State Space Duality and Mamba-2" ("The SSD Block Decomposition
// Algorithm"): the diagonal block of chunk c is ((C_c B_c^T) o L) X_c, and
// C_c B_c^T depends on the group only, not on the head; the same page
// ("Multi-Head SSM Patterns") shares B and C across the heads of a group in
// the manner of grouped-query attention.  This kernel evaluates the lower
// triangle of C_c B_c^T once per group on MFMA (fp32 accumulation, rounded
// to bf16 for the head kernels) and also writes B_c token-transposed, the
// operand layout of the chunk-state contraction B_c^T diag(w dt) X_c.
//
// Both are written in the exact per-lane order in which the chunk kernel
// loads them as MFMA operands (16 bytes per lane, 1 KB per wave load):
//
//   S block (I, m), m <= I/2, for 16-token row tile I and 32-token pair m:
//     lane l (i = 16 I + l%16, g = l/16), element e = 0..7 holds
//     (C_c B_c^T)[i][j] at j = 32 m + 4 g + (e % 4) + 16 (e / 4);
//     blocks are stored row tile by row tile, I ascending, m ascending.
//   B^T fragment (m, n): 4 x 16 bytes, part g holds B_c[j][n] at the same
//     8 tokens j(e, g).
//   C fragment (I, kk): lane l holds C_c[16 I + l%16][32 kk + 8 (l/16) .. +7]
//     (the B operand of the state projection), written by block (I, 0).
//
// Tokens past the end of the row read as zero.
#include "ssd_common.hpp"

namespace ssd {

// One wave per work item of a (batch row, group, chunk): items 0 .. NBLK-1
// are the C B^T blocks (I, m) in storage order, items NBLK .. NBLK+NP*N/16-1
// the B^T fragments (pair m, 16-column n-tile).  Four items per workgroup.
template <int Q, int N>
struct CbItems {
    static constexpr int NTILE = N / 16;
    static constexpr int COUNT = CbShape<Q>::NBLK + CbShape<Q>::NP * NTILE;
};

template <int Q, int N>
__global__ __launch_bounds__(256) void ssd_cb_kernel(CbArgs a) {
    using S = CbShape<Q>;
    constexpr int KN = (N >= 32) ? N / 32 : 1;
    constexpr int ITEMS = CbItems<Q, N>::COUNT, NTILE = CbItems<Q, N>::NTILE;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const int64_t item_all = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nitems = (int64_t)a.batch * a.ngroups * a.nchunks * ITEMS;
    if (item_all >= nitems) return;
    const int item = (int)(item_all % ITEMS);
    const int64_t bgc = item_all / ITEMS;        // (b * G + grp) * nchunks + c
    const int c = (int)(bgc % a.nchunks);
    const int64_t bg = bgc / a.nchunks;
    const int grp = (int)(bg % a.ngroups), b = (int)(bg / a.ngroups);
    const int L = a.seqlen, G = a.ngroups;
    const int t0 = c * Q;
    const bf16 *Bsrc = (const bf16 *)a.B + ((int64_t)b * L * G + grp) * N;
    const bf16 *Csrc = (const bf16 *)a.C + ((int64_t)b * L * G + grp) * N;
    auto row8 = [&](const bf16 *src, int t, int col) -> bf16x8 {
        if (t >= L || col >= N) return bf16x8{};
        return *(const bf16x8 *)(src + (int64_t)t * G * N + col);
    };

    if (item < S::NBLK) {
        // block (I, m): the row tile I with off(I) <= item < off(I + 1)
        int I = 0;
        while (I + 1 < S::TILES && S::off(I + 1) <= item) ++I;
        const int m = item - S::off(I);
        bf16x8 cf[KN];
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) cf[kk] = row8(Csrc, t0 + 16 * I + l16, kk * 32 + 8 * g);
        if (m == 0) {
#pragma unroll
            for (int kk = 0; kk < KN; ++kk)
                ((bf16x8 *)a.ws_C)[((bgc * S::TILES + I) * KN + kk) * 64 + lane] = cf[kk];
        }
        f32x4 d[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int J = 2 * m + h;
            if (J > I) continue;
            bf16x8 bfr[KN];
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) bfr[kk] = row8(Bsrc, t0 + 16 * J + l16, kk * 32 + 8 * g);
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) d[h] = mfma_bf16(bfr[kk], cf[kk], d[h]);
        }
        mfma_fence(d[0], d[1]);
        bf16x8 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            o[r] = (bf16)d[0][r];
            o[4 + r] = (bf16)d[1][r];
        }
        ((bf16x8 *)a.ws_S)[(bgc * S::NBLK + item) * 64 + lane] = o;
    } else {
        // B^T fragment (pair k, n-tile nt): lane (l16, g) gathers B[t][n] at
        // n = 16 nt + l16 for its 8 slot tokens (16 lanes read 32 contiguous
        // bytes of one token row per load), all loads in one round trip
        const int k = (item - S::NBLK) / NTILE, nt = (item - S::NBLK) % NTILE;
        const int n = 16 * nt + l16;
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = t0 + 32 * k + 4 * g + (e & 3) + 16 * (e >> 2);
            v[e] = (t < L) ? Bsrc[(int64_t)t * G * N + n] : (bf16)0.f;
        }
        ((bf16x8 *)a.ws_BT)[((bgc * S::NP + k) * N + n) * 4 + g] = v;
    }
}

size_t cb_s_elems(int Q) {
    switch (Q) {
    case 64: return (size_t)CbShape<64>::NBLK * 64 * 8;
    case 128: return (size_t)CbShape<128>::NBLK * 64 * 8;
    default: return (size_t)CbShape<256>::NBLK * 64 * 8;
    }
}

#define SSD_CB_CASE(q, n)                                                                   \
    if (Q == q && N == n) {                                                                 \
        constexpr int items = CbItems<q, n>::COUNT;                                          \
        const int64_t total = (int64_t)a.batch * a.ngroups * a.nchunks * items;              \
        hipLaunchKernelGGL((ssd_cb_kernel<q, n>), dim3((unsigned)((total + 3) / 4)), dim3(256), \
                           0, stream, a);                                                   \
        return true;                                                                        \
    }

bool launch_cb(int Q, int N, const CbArgs &a, hipStream_t stream) {
    SSD_CB_CASE(64, 16) SSD_CB_CASE(64, 32) SSD_CB_CASE(64, 64) SSD_CB_CASE(64, 128)
    SSD_CB_CASE(128, 16) SSD_CB_CASE(128, 32) SSD_CB_CASE(128, 64) SSD_CB_CASE(128, 128)
    SSD_CB_CASE(256, 16) SSD_CB_CASE(256, 32) SSD_CB_CASE(256, 64) SSD_CB_CASE(256, 128)
    return false;
}

}  // namespace ssd
