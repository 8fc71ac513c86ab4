// Backward pass of the SSD forward pass (gradients of every input), fp32 on
// the vector ALU, chunk by chunk in reverse.
//
// With the chunk-entering states H_{c-1} (from the forward machinery's
// split-local pass and affine scan, one split per 64-token chunk) and the
// adjoint G_c = dJ/dH_c of the state at the end of chunk c, everything a
// chunk contributes is a masked quadratic form plus state terms (page "State
// Space Duality and Mamba-2", "The SSD Block Decomposition Algorithm", read
// backwards).  Per chunk of Q tokens, with L the decay mask, S = C B^T,
// V = dY X^T (P contraction), u_i the decay from the chunk start through i,
// w_j the decay from j to the chunk end and T the chunk decay:
//
//   dX_j   = sum_{i>=j} L_ij S_ij dy_i + w_j G B_j          (w.r.t. dt_j x_j)
//   dx_j   = dt_j dX_j + D dy_j
//   dB_j   = dt_j sum_{i>=j} L_ij V_ij C_i + w_j dt_j G^T x_j
//   dC_i   = sum_{j<=i} L_ij dt_j V_ij B_j + u_i H^T dy_i
//   dl_t   = sum_{s>=t>r} R_sr + sum_{s>=t} q_s + sum_{r<t} p_r + T <G, H>
//            R = L o dt o S o V,  q_s = u_s dy_s^T H C_s,  p_r = w_r dt_r x_r^T G B_r
//   ddt_t  = x_t . dX_t + A dl_t,    dA += sum_t dt_t dl_t,    dD += sum_t dy_t . x_t
//   G_{c-1} = T G_c + sum_i u_i dy_i C_i^T
//
// where dl_t = a_t <g_t, h_{t-1}> is the gradient through the log-decay of
// token t (zero at a document boundary: every factor spanning it is 0).  The
// mask is evaluated row by row as nested sums leftwards from the diagonal
// (values in [0, 1], non-increasing away from the diagonal).  One workgroup
// per (batch row, head); dB and dC are written per head and summed over the
// heads of a group by ssd_bwd_reduce_kernel, as are dA and dD over rows.
#include "ssd_common.hpp"
#include "ssd_segsum.hpp"

namespace ssd {

template <typename IO>
__device__ inline float bwd_ld(const void *p, int64_t i) {
    return (float)((const IO *)p)[i];
}

// 16 waves: one workgroup fills a CU (its LDS allows one per CU), so that
// four waves per SIMD cover the latency of the global-memory operands.
constexpr int kBwdThreads = 1024;

template <typename IO>
__global__ __launch_bounds__(kBwdThreads, 1) void ssd_bwd_kernel(BwdArgs a) {
    constexpr int Q = kBwdQ, NB = Q / 16;
    constexpr int LQ = Q + 1;               // padded row pitch: a lane per row hits its own bank
    constexpr int kMaxPN = 128 * 128;
    __shared__ __attribute__((aligned(16))) SegLds<Q> sg;
    __shared__ float sG[kMaxPN];           // adjoint of the state at the chunk end, [P][N]
    __shared__ float sL[Q * LQ];            // decay mask L[i][j]
    __shared__ float sS[Q * LQ];            // (C B^T)[i][j]
    __shared__ float sR[Q * LQ];            // V[i][j] = dy_i . x_j, then R, then row prefix sums of R
    __shared__ float sT[Q * 129];           // staged rows of B, then of x (pitch +1)
    __shared__ float sw[Q];                 // decay from token j to the chunk end
    __shared__ float sq[Q], sp[Q], sxdX[Q], sdl[Q];
    __shared__ float sK, sDD, sDA;

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / a.nheads, h = bh % a.nheads;
    const int L = a.seqlen, H = a.nheads, G = a.ngroups, P = a.headdim, N = a.dstate;
    const int PN = P * N;
    const int grp = h / (H / G);
    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.f;
    const float *dt_row = a.dt + (int64_t)b * L * H + h;
    const int32_t *seq_row = a.seq_idx ? a.seq_idx + (int64_t)b * L : nullptr;
    auto xi = [&](int t, int p) { return bwd_ld<IO>(a.x, (((int64_t)b * L + t) * H + h) * P + p); };
    auto dyi = [&](int t, int p) { return bwd_ld<IO>(a.dy, (((int64_t)b * L + t) * H + h) * P + p); };
    auto Bi = [&](int t, int n) { return bwd_ld<IO>(a.B, (((int64_t)b * L + t) * G + grp) * N + n); };
    auto Ci = [&](int t, int n) { return bwd_ld<IO>(a.C, (((int64_t)b * L + t) * G + grp) * N + n); };

    for (int e = tid; e < PN; e += kBwdThreads)
        sG[e] = a.dfinal ? a.dfinal[(int64_t)bh * PN + e] : 0.f;
    if (tid == 0) {
        sDD = 0.f;
        sDA = 0.f;
    }
    __syncthreads();

    for (int c = a.nchunks - 1; c >= 0; --c) {
        const int t0 = c * Q;
        const int nvalid = min(Q, L - t0);
        // H_{c-1}: from the forward's scan, or (a single chunk) the initial state or 0
        const float *Hs = a.states ? a.states + ((int64_t)bh * a.nchunks + c) * PN
                                   : (a.init_states ? a.init_states + (int64_t)bh * PN : nullptr);

        // ---- segsum values of the chunk (the forward kernels' helpers)
        int flag_any = 0;
        if (tid < Q) {
            seg_load_token<Q>(sg, tid, t0, nvalid, dt_row, H, A_h, seq_row, dt_map_identity());
            flag_any = sg.flag[tid];
        }
        flag_any = __syncthreads_or(flag_any);
        if (tid == 0) {
            sg.any_reset = flag_any;
            sK = 0.f;
        }
        if (tid < Q) seg_block_sums<Q>(sg, tid);
        __syncthreads();
        if (tid < Q) {
            seg_chunk_products<Q>(sg, tid);
            const int K = tid >> 4;
            float Z = 1.f;
            for (int k = NB - 1; k > K; --k) Z = __fmul_rn(Z, sg.Tb[k]);
            sw[tid] = __fmul_rn(sg.W[tid], Z);
            sq[tid] = 0.f;
            sp[tid] = 0.f;
            sxdX[tid] = 0.f;
        }
        __syncthreads();

        // ---- mask rows (nested sums leftwards from the diagonal), S and V
        if (tid < Q) {
            const int i = tid;
            float sum = 0.f;
            for (int j = i; j >= 0; --j) {
                float v = (sg.rs[i] > j) ? 0.f : __builtin_amdgcn_exp2f(sum);
                if (i >= nvalid) v = 0.f;
                sL[i * LQ + j] = v;
                sum = __fadd_rn(sum, sg.d[j]);
            }
            for (int j = i + 1; j < Q; ++j) sL[i * LQ + j] = 0.f;
        }
        // S = C B^T with B's rows staged in LDS (the lanes of a wave take
        // different j), then V = dY X^T with x's rows staged in the same place
        for (int e = tid; e < Q * N; e += kBwdThreads) {
            const int j = e / N, n = e % N;
            sT[j * (N + 1) + n] = (j < nvalid) ? Bi(t0 + j, n) : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < Q * Q; e += kBwdThreads) {
            const int i = e / Q, j = e % Q;
            float s = 0.f;
            if (j <= i && i < nvalid)
                
#pragma unroll 8
                for (int n = 0; n < N; ++n) s = fmaf(Ci(t0 + i, n), sT[j * (N + 1) + n], s);
            sS[i * LQ + j] = s;
        }
        __syncthreads();
        for (int e = tid; e < Q * P; e += kBwdThreads) {
            const int j = e / P, p = e % P;
            sT[j * (P + 1) + p] = (j < nvalid) ? xi(t0 + j, p) : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < Q * Q; e += kBwdThreads) {
            const int i = e / Q, j = e % Q;
            float v = 0.f;
            if (j <= i && i < nvalid)
                
#pragma unroll 8
                for (int p = 0; p < P; ++p) v = fmaf(dyi(t0 + i, p), sT[j * (P + 1) + p], v);
            sR[i * LQ + j] = v;
        }
        __syncthreads();

        // ---- dX (and x . dX, p_r), dx, and dy . x for dD
        float ddsum = 0.f;
        for (int e = tid; e < Q * P; e += kBwdThreads) {
            const int j = e / P, p = e % P;
            if (j >= nvalid) continue;
            float acc = 0.f;
            
#pragma unroll 8
                for (int i = j; i < nvalid; ++i) acc = fmaf(sL[i * LQ + j] * sS[i * LQ + j], dyi(t0 + i, p), acc);
            float gb = 0.f;
            
#pragma unroll 8
                for (int n = 0; n < N; ++n) gb = fmaf(sG[p * N + n], Bi(t0 + j, n), gb);
            const float dX = fmaf(sw[j], gb, acc);
            const float xv = xi(t0 + j, p);
            const float dtj = sg.dt[j];
            const float dyv = dyi(t0 + j, p);
            a.dx[(((int64_t)b * L + t0 + j) * H + h) * P + p] = fmaf(dtj, dX, D_h * dyv);
            atomicAdd(&sxdX[j], xv * dX);
            ddsum = fmaf(dyv, xv, ddsum);
            atomicAdd(&sp[j], sg.wcd[j] * xv * gb);
        }
        // ---- dB (per head), dC (per head) and q_s
        for (int e = tid; e < Q * N; e += kBwdThreads) {
            const int t = e / N, n = e % N;
            if (t >= nvalid) continue;
            // dB_t: column t of the masked products, and the state term
            float accb = 0.f;
            
#pragma unroll 8
                for (int i = t; i < nvalid; ++i) accb = fmaf(sL[i * LQ + t] * sR[i * LQ + t], Ci(t0 + i, n), accb);
            float gx = 0.f;
            
#pragma unroll 8
                for (int p = 0; p < P; ++p) gx = fmaf(sG[p * N + n], xi(t0 + t, p), gx);
            const float dtt = sg.dt[t];
            a.dB_head[(((int64_t)b * L + t0 + t) * H + h) * N + n] = dtt * fmaf(sw[t], gx, accb);
            // dC_t: row t of the masked products, and the state term
            float accc = 0.f;
            
#pragma unroll 8
                for (int j = 0; j <= t; ++j) accc = fmaf(sL[t * LQ + j] * sg.dt[j] * sR[t * LQ + j], Bi(t0 + j, n), accc);
            float hdy = 0.f;
            if (Hs)
                
#pragma unroll 8
                for (int p = 0; p < P; ++p) hdy = fmaf(Hs[p * N + n], dyi(t0 + t, p), hdy);
            a.dC_head[(((int64_t)b * L + t0 + t) * H + h) * N + n] = fmaf(sg.u[t], hdy, accc);
            atomicAdd(&sq[t], sg.u[t] * hdy * Ci(t0 + t, n));
        }
        atomicAdd(&sDD, ddsum);
        // ---- T <G, H>
        {
            float k = 0.f;
            if (Hs)
                for (int e = tid; e < PN; e += kBwdThreads) k = fmaf(sG[e], Hs[e], k);
            atomicAdd(&sK, k);
        }
        __syncthreads();

        // ---- R = L o dt o S o V, then prefix sums of each row over r < t
        if (tid < Q) {
            const int s = tid;
            float run = 0.f;
            for (int r = 0; r < Q; ++r) {
                const float R = (r <= s) ? sL[s * LQ + r] * sg.dt[r] * sS[s * LQ + r] * sR[s * LQ + r] : 0.f;
                sR[s * LQ + r] = run;          // sum_{r' < r} R_{s r'}
                run += R;
            }
        }
        __syncthreads();
        if (tid < Q) {
            const int t = tid;
            float dl = 0.f;
            if (t < nvalid) {
                for (int s = t; s < Q; ++s) dl += sR[s * LQ + t] + sq[s];
                for (int r = 0; r < t; ++r) dl += sp[r];
                dl += sg.T * sK;
                if (sg.flag[t]) dl = 0.f;   // a_t is 0 there, not exp(dt A)
                a.ddt[((int64_t)b * L + t0 + t) * H + h] = fmaf(A_h, dl, sxdX[t]);
            }
            sdl[t] = (t < nvalid) ? sg.dt[t] * dl : 0.f;
        }
        __syncthreads();
        if (tid == 0) {
            float s = 0.f;
            for (int t = 0; t < Q; ++t) s += sdl[t];
            sDA += s;
        }
        // ---- G_{c-1} = T G_c + sum_i u_i dy_i C_i^T
        for (int e = tid; e < PN; e += kBwdThreads) {
            const int p = e / N, n = e % N;
            float acc = sg.T * sG[e];
            
#pragma unroll 8
                for (int i = 0; i < nvalid; ++i) acc = fmaf(sg.u[i] * dyi(t0 + i, p), Ci(t0 + i, n), acc);
            sG[e] = acc;
        }
        __syncthreads();
    }
    if (a.dinit)
        for (int e = tid; e < PN; e += kBwdThreads) a.dinit[(int64_t)bh * PN + e] = sG[e];
    if (tid == 0) {
        a.dA_part[bh] = sDA;
        a.dD_part[bh] = sDD;
    }
}

// dB, dC [b][L][G][N] = sum over the heads of each group of the per-head
// values; dA, dD [H] = sum over batch rows.  One thread per output element.
__global__ __launch_bounds__(256) void ssd_bwd_reduce_kernel(BwdArgs a) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int H = a.nheads, G = a.ngroups, N = a.dstate, hpg = H / G;
    const int64_t nbg = (int64_t)a.batch * a.seqlen * G * N;
    if (e < nbg) {
        const int n = (int)(e % N);
        const int64_t r = e / N;
        const int g = (int)(r % G);
        const int64_t bt = r / G;
        float sb = 0.f, sc = 0.f;
        for (int k = 0; k < hpg; ++k) {
            const int64_t o = (bt * H + g * hpg + k) * N + n;
            sb += a.dB_head[o];
            sc += a.dC_head[o];
        }
        a.dB[e] = sb;
        a.dC[e] = sc;
    } else if (e < nbg + H) {
        const int h = (int)(e - nbg);
        float sa = 0.f, sd = 0.f;
        for (int bb = 0; bb < a.batch; ++bb) {
            sa += a.dA_part[(int64_t)bb * H + h];
            sd += a.dD_part[(int64_t)bb * H + h];
        }
        a.dA[h] = sa;
        if (a.dD) a.dD[h] = sd;
    }
}

void launch_bwd(bool bf16_io, const BwdArgs &a, hipStream_t stream) {
    const dim3 grid(a.batch * a.nheads), block(kBwdThreads);
    if (bf16_io) hipLaunchKernelGGL(ssd_bwd_kernel<bf16>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(ssd_bwd_kernel<float>, grid, block, 0, stream, a);
    const int64_t total = (int64_t)a.batch * a.seqlen * a.ngroups * a.dstate + a.nheads;
    hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, a);
}

}  // namespace ssd
