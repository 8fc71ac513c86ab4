// fp32 chunk kernel of the SSD forward pass (vector ALU, fp32 throughout).
//
// The precision path for fp32 inputs: the same chunked algorithm, segsum
// and split structure as the bf16 MFMA kernel, with every product and sum in
// fp32.  One workgroup owns one (batch row, head, split) and walks its
// chunks; per chunk (page "State Space Duality and Mamba-2", "The SSD Block
// Decomposition Algorithm"):
//   for each 16-row strip of the chunk:
//     M[i][j] = (C_i . B_j) L_ij dt_j            masked diagonal block, in LDS
//     y_i     = u_i h_{c-1} C_i + sum_j M[i][j] x_j + D x_i
//   h_c = T_c h_{c-1} + sum_j (w_j dt_j) x_j B_j^T
// With the fused prologue, dt is mapped from the raw values as it is loaded
// (bias, softplus, clamp); with the fused gate, y_i is multiplied by
// silu(z_i) as it is stored.
// The mask L comes from the same segsum device functions as the bf16 kernel
// (ssd_segsum.hpp), evaluated row by row.
#include "ssd_common.hpp"
#include "ssd_segsum.hpp"

namespace ssd {

// VARIANT selects how the intra-chunk mask entries are evaluated (tests and
// benchmarks of page "GPU Hierarchy Meets Structured Matrices", abstract):
// the hierarchy-aware segsum of the other kernels, the dense direct segsum
// (each entry its own sum over (j, i]) or the diff segsum (2^(cs_i - cs_j)
// from prefix sums cs of an associative scan).  Only the mask L varies; the
// state decays u, w and T come from the same sub-block products in all three.
template <int Q, int VARIANT>
__global__ __launch_bounds__(kThreads, 1) void ssd_chunk_f32_kernel(ChunkArgs a) {
    constexpr int NB = Q / 16;
    constexpr int kMaxPN = 128 * 128;
    __shared__ __attribute__((aligned(16))) SegLds<Q> sg;
    __shared__ float cs[Q];             // prefix sums (diff segsum only)
    __shared__ float sH[kMaxPN];        // state, [P][N]
    __shared__ float sM[16 * Q];        // masked strip of the diagonal block
    __shared__ float sRowF[16 * NB];    // F(i, J) of the strip's rows
    __shared__ float sRowD[16 * 16];    // diagonal sub-block mask values

    const int tid = threadIdx.x;
    const Unit un = unit_of_block(a, (int)blockIdx.x);
    const int b = un.b, h = un.h, s = un.s;
    if (a.mode == kModeSplitLocal && s == a.nsplits - 1) return;
    const int L = a.seqlen, H = a.nheads, G = a.ngroups, P = a.headdim, N = a.dstate;
    const int PN = P * N;
    const int grp = h / (H / G);
    const bool full = a.mode == kModeFull;
    const int c_begin = s * a.split_chunks;
    const int c_end = min(a.nchunks, c_begin + a.split_chunks);
    const float *xg = (const float *)a.x;
    const float *Bg = (const float *)a.B;
    const float *Cg = (const float *)a.C;
    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.f;
    const float *dt_row = a.dt + (int64_t)b * L * H + h;
    const DtMap dm = dt_map_of(a, h);
    const float *zg = (const float *)a.z;
    const int32_t *seq_row = a.seq_idx ? a.seq_idx + (int64_t)b * L : nullptr;
    auto xrow = [&](int t) { return xg + (((int64_t)b * L + t) * H + h) * P; };
    auto brow = [&](int t) { return Bg + (((int64_t)b * L + t) * G + grp) * N; };
    auto crow = [&](int t) { return Cg + (((int64_t)b * L + t) * G + grp) * N; };

    {
        const float *src = nullptr;
        if (full && s == 0) src = a.init_states ? a.init_states + ((int64_t)b * H + h) * PN : nullptr;
        else if (full) src = a.ws_states + (((int64_t)b * H + h) * a.nsplits + s) * PN;
        for (int e = tid; e < PN; e += kThreads) sH[e] = src ? src[e] : 0.f;
    }
    float split_decay = 1.f;

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * Q;
        const int nvalid = min(Q, L - t0);
        int flag_any = 0;
        if (tid < Q) {
            seg_load_token<Q>(sg, tid, t0, nvalid, dt_row, H, A_h, seq_row, dm);
            flag_any = sg.flag[tid];
        }
        flag_any = __syncthreads_or(flag_any);
        if (tid == 0) sg.any_reset = flag_any;
        if (tid < Q) seg_block_sums<Q>(sg, tid);
        __syncthreads();
        if (tid < Q) seg_chunk_products<Q>(sg, tid);
        __syncthreads();
        if constexpr (VARIANT == kSegsumDiff) {
            // inclusive prefix sums of the log2-decays by a Kogge-Stone scan
            if (tid < Q) cs[tid] = sg.d[tid];
            __syncthreads();
            for (int off = 1; off < Q; off *= 2) {
                const float v = (tid < Q && tid >= off) ? cs[tid - off] : 0.f;
                __syncthreads();
                if (tid < Q && tid >= off) cs[tid] = __fadd_rn(cs[tid], v);
                __syncthreads();
            }
        }

        if (full) {
            for (int I = 0; I < NB; ++I) {
                const int I0 = I * 16;
                if (VARIANT == kSegsumHierarchy && tid < 16) {
                    const int i = I0 + tid;
                    const int rs_i = sg.rs[i];
                    float e[4];
                    float sum0 = 0.f;
                    for (int gg = 0; gg < 4; ++gg) {
                        sum0 = seg_diag_row(sg.d, I0, i, gg, e);
                        for (int r = 0; r < 4; ++r)
                            sRowD[tid * 16 + 4 * gg + r] = seg_diag_value(e[r], i, I0 + 4 * gg + r, rs_i);
                    }
                    float F = seg_chain_start(sum0, I0, rs_i);
                    for (int J = I - 1; J >= 0; --J) {
                        if (J < I - 1) F = seg_chain_step(F, sg.Tb[J + 1]);
                        sRowF[tid * NB + J] = F;
                    }
                }
                __syncthreads();
                const int ncol = I0 + 16;
                for (int e = tid; e < 16 * ncol; e += kThreads) {
                    const int ii = e / ncol, j = e % ncol;
                    const int i = I0 + ii;
                    float v = 0.f;
                    if (i < nvalid && j <= i) {
                        float Lij;
                        if constexpr (VARIANT == kSegsumDirect) {
                            float run = 0.f;
                            for (int k = j + 1; k <= i; ++k) run = __fadd_rn(run, sg.d[k]);
                            Lij = (sg.rs[i] > j) ? 0.f : __builtin_amdgcn_exp2f(run);
                        } else if constexpr (VARIANT == kSegsumDiff) {
                            Lij = (sg.rs[i] > j) ? 0.f : __builtin_amdgcn_exp2f(__fsub_rn(cs[i], cs[j]));
                        } else {
                            const int J = j >> 4;
                            Lij = (J == I) ? sRowD[ii * 16 + (j & 15)]
                                           : seg_offdiag(sRowF[ii * NB + J], sg.W[j]);
                        }
                        const float *ci = crow(t0 + i), *bj = brow(t0 + j);
                        float dot = 0.f;
                        for (int n = 0; n < N; ++n) dot = fmaf(ci[n], bj[n], dot);
                        v = dot * Lij * sg.dt[j];
                    }
                    sM[ii * Q + j] = v;
                }
                __syncthreads();
                for (int e = tid; e < 16 * P; e += kThreads) {
                    const int ii = e / P, p = e % P;
                    const int i = I0 + ii;
                    if (i >= nvalid) continue;
                    const float *ci = crow(t0 + i);
                    const float *hp = sH + p * N;
                    float proj = 0.f;
                    for (int n = 0; n < N; ++n) proj = fmaf(ci[n], hp[n], proj);
                    float acc = proj * sg.u[i];
                    for (int j = 0; j <= i; ++j) acc = fmaf(sM[ii * Q + j], xrow(t0 + j)[p], acc);
                    const float xi = xrow(t0 + i)[p];
                    const int64_t o = (((int64_t)b * L + t0 + i) * H + h) * P + p;
                    float out = acc + D_h * xi;
                    // output gate (element-wise, after the skip term)
                    if (zg) out = out * silu_f32(zg[o]);
                    ((float *)a.y)[o] = out;
                }
                __syncthreads();
            }
        }

        const float Tc = sg.T;
        split_decay = __fmul_rn(split_decay, Tc);
        for (int e = tid; e < PN; e += kThreads) {
            const int p = e / N, n = e % N;
            float acc = sH[e] * Tc;
            for (int j = 0; j < nvalid; ++j) acc = fmaf(sg.wcd[j] * xrow(t0 + j)[p], brow(t0 + j)[n], acc);
            sH[e] = acc;
        }
        __syncthreads();
    }

    float *dst = nullptr;
    if (full) {
        if (s == a.nsplits - 1 && a.final_states) dst = a.final_states + ((int64_t)b * H + h) * PN;
    } else {
        dst = a.ws_states + (((int64_t)b * H + h) * a.nsplits + s) * PN;
        if (tid == 0) a.ws_decay[((int64_t)b * H + h) * a.nsplits + s] = split_decay;
    }
    if (dst)
        for (int e = tid; e < PN; e += kThreads) dst[e] = sH[e];
}

template <int VARIANT>
static void launch_chunk_f32_v(int Q, const ChunkArgs &a, hipStream_t stream) {
    const dim3 grid(a.units), block(kThreads);
    switch (Q) {
    case 64: hipLaunchKernelGGL((ssd_chunk_f32_kernel<64, VARIANT>), grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((ssd_chunk_f32_kernel<128, VARIANT>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((ssd_chunk_f32_kernel<256, VARIANT>), grid, block, 0, stream, a); break;
    }
}

void launch_chunk_f32(int Q, const ChunkArgs &a, hipStream_t stream) {
    switch (a.segsum_variant) {
    case kSegsumDirect: launch_chunk_f32_v<kSegsumDirect>(Q, a, stream); break;
    case kSegsumDiff: launch_chunk_f32_v<kSegsumDiff>(Q, a, stream); break;
    default: launch_chunk_f32_v<kSegsumHierarchy>(Q, a, stream); break;
    }
}

}  // namespace ssd
