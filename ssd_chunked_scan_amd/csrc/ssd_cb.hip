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
#include "ssd_tiles.hpp"

namespace ssd {

// Work split: NQ = Q/64 workgroups per (batch row, group, chunk).  Workgroup
// k owns the row tiles {k, 2NQ-1-k, 2NQ+k, 4NQ-1-k} (the same number of C B^T
// blocks for every k) and the B^T fragments of pairs [k NP/NQ, (k+1) NP/NQ).
// It stages the chunk's B rows and its own four C row tiles in LDS with
// direct loads (each global byte read once per workgroup), then every
// operand is an LDS read.
template <int Q, int N>
struct CbCfg {
    static constexpr int NQ = Q / 64;          // workgroups per chunk
    static constexpr int TILES = Q / 16, NP = Q / 32;
    static constexpr int KN = (N >= 32) ? N / 32 : 1;
    static constexpr int CPR = N / 8;          // 16-byte chunks per B or C row
    static constexpr int NT = N / 16;          // n-tiles
    static constexpr int PPW = NP / NQ;        // B^T pairs per workgroup
};

template <int Q, int N>
__global__ __launch_bounds__(256) void ssd_cb_kernel(CbArgs a) {
    using S = CbShape<Q>;
    using Cfg = CbCfg<Q, N>;
    constexpr int NQ = Cfg::NQ, TILES = Cfg::TILES, KN = Cfg::KN, CPR = Cfg::CPR, NT = Cfg::NT;
    constexpr int PPW = Cfg::PPW;
    // B rows of the chunk and the workgroup's 4 C row tiles, swizzled rows of
    // CPR 16-byte chunks
    __shared__ __attribute__((aligned(1024))) bf16 sB[Q * N];
    __shared__ __attribute__((aligned(1024))) bf16 sC[64 * N];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int k = (int)(blockIdx.x % NQ);
    const int64_t bgc = blockIdx.x / NQ;         // (b * G + grp) * nchunks + c
    const int c = (int)(bgc % a.nchunks);
    const int64_t bg = bgc / a.nchunks;
    const int grp = (int)(bg % a.ngroups), b = (int)(bg / a.ngroups);
    const int L = a.seqlen, G = a.ngroups, t0 = c * Q;
    const int nvalid = min(Q, L - t0);
    const bf16 *Bsrc = (const bf16 *)a.B + (((int64_t)b * L + t0) * G + grp) * N;
    const bf16 *Csrc = (const bf16 *)a.C + (((int64_t)b * L + t0) * G + grp) * N;
    auto tile_of = [&](int ti) __attribute__((always_inline)) {
        return ti == 0 ? k : ti == 1 ? 2 * NQ - 1 - k : ti == 2 ? 2 * NQ + k : 4 * NQ - 1 - k;
    };

    // ---- staging: whole 1 KB blocks of 64 16-byte chunks, 4 waves
    {
        constexpr int nbB = Q * CPR / 64;
        for (int blk = wave; blk < nbB; blk += 4) {
            const int slot = blk * 64 + lane, r = slot / CPR, pc = slot % CPR;
            const int cc = pc ^ swz<CPR>(r);
            const bf16 *src = (r < nvalid) ? Bsrc + (int64_t)r * G * N + cc * 8 : kZeroChunk;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(sB + blk * 512), 16, 0, 0);
        }
        constexpr int nbC = 64 * CPR / 64;
        for (int blk = wave; blk < nbC; blk += 4) {
            const int slot = blk * 64 + lane, r = slot / CPR, pc = slot % CPR;   // r: row of the 4 staged tiles
            const int cc = pc ^ swz<CPR>(r);
            const int t = tile_of(r >> 4) * 16 + (r & 15);
            const bf16 *src = (t < nvalid) ? Csrc + (int64_t)t * G * N + cc * 8 : kZeroChunk;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(sC + blk * 512), 16, 0, 0);
        }
        vmem_lds_sync();
    }
    // 8 k-consecutive bf16 of a staged row at column col (a multiple of 8),
    // zero past dstate
    auto row8 = [&](const bf16 *tile, int r, int col) __attribute__((always_inline)) -> bf16x8 {
        if (col >= N) return bf16x8{};
        return *(const bf16x8 *)&tile[tile_off<CPR>(r, col >> 3)];
    };

    // ---- C B^T blocks (I, m) of the 4 row tiles, dealt to the waves in turn
    {
        int q = 0;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int I = tile_of(ti);
            for (int m = 0; m <= I / 2; ++m, ++q) {
                if (q % 4 != wave) continue;
                bf16x8 cf[KN];
#pragma unroll
                for (int kk = 0; kk < KN; ++kk) cf[kk] = row8(sC, ti * 16 + l16, kk * 32 + 8 * g);
                f32x4 d[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int J = 2 * m + h;
                    if (J > I) continue;
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk)
                        d[h] = mfma_bf16(row8(sB, J * 16 + l16, kk * 32 + 8 * g), cf[kk], d[h]);
                }
                mfma_fence(d[0], d[1]);
                bf16x8 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    o[r] = (bf16)d[0][r];
                    o[4 + r] = (bf16)d[1][r];
                }
                ((bf16x8 *)a.ws_S)[(bgc * S::NBLK + S::off(I) + m) * 64 + lane] = o;
            }
        }
    }
    // ---- C fragments (I, kk) of the 4 row tiles
    for (int f = wave; f < 4 * KN; f += 4) {
        const int ti = f / KN, kk = f % KN;
        ((bf16x8 *)a.ws_C)[((bgc * TILES + tile_of(ti)) * KN + kk) * 64 + lane] =
            row8(sC, ti * 16 + l16, kk * 32 + 8 * g);
    }
    // ---- B^T fragments (pair m, n-tile nt): lane (l16, g) holds B[j][n] at
    // n = 16 nt + l16 for its 8 slot tokens j, by 16-bit transpose reads
    for (int f = wave; f < PPW * NT; f += 4) {
        const int m = k * PPW + f / NT, nt = f % NT;
        const int rr = 32 * m + 4 * g + (l16 >> 2), col = nt * 16 + 4 * (l16 & 3);
        const bf16x8 v = join_bf16x8(lds_read_tr16(&sB[tile_off_col<CPR>(rr, col)]),
                                     lds_read_tr16(&sB[tile_off_col<CPR>(rr + 16, col)]));
        ((bf16x8 *)a.ws_BT)[((bgc * S::NP + m) * N + nt * 16 + l16) * 4 + g] = v;
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
        const int64_t total = (int64_t)a.batch * a.ngroups * a.nchunks * CbCfg<q, n>::NQ;   \
        hipLaunchKernelGGL((ssd_cb_kernel<q, n>), dim3((unsigned)total), dim3(256), 0, stream, a); \
        return true;                                                                        \
    }

bool launch_cb(int Q, int N, const CbArgs &a, hipStream_t stream) {
    SSD_CB_CASE(64, 16) SSD_CB_CASE(64, 32) SSD_CB_CASE(64, 64) SSD_CB_CASE(64, 128)
    SSD_CB_CASE(128, 16) SSD_CB_CASE(128, 32) SSD_CB_CASE(128, 64) SSD_CB_CASE(128, 128)
    SSD_CB_CASE(256, 16) SSD_CB_CASE(256, 32) SSD_CB_CASE(256, 64) SSD_CB_CASE(256, 128)
    return false;
}

}  // namespace ssd
