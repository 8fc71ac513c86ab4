// bf16 chunk kernel of the SSD forward pass on gfx950 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// One workgroup (4 wave64s) owns one (batch row, head, sequence split,
// headdim block) and walks the split's chunks in order, carrying the N x P
// state in fp32 registers (page "NVIDIA Accelerates Mamba-2 Forward Kernel
// with CUDA Tile", "What CUDA Tile Is": tile by tile with the state kept on
// chip).  Per chunk c of Q tokens (page "State Space Duality and Mamba-2",
// "The SSD Block Decomposition Algorithm"):
//
//   segsum      decay factors and mask of the chunk (ssd_segsum.hpp)
//   output      Y^T = (h_{c-1}^T C_c^T) diag(u)            state projection
//                   + X_c^T ((C_c B_c^T) o L o dt)^T          diagonal block
//                   + D x_c                                    skip
//   state       h_c = T_c h_{c-1} + B_c^T diag(w dt) X_c       chunk state
//
// Everything is computed transposed (rows = headdim p) so that each lane of
// an output tile owns one token i and four consecutive p: the row scale u_i
// is one value per lane and y is written 8 bytes per lane.
//
// MFMA 16x16x32 bf16 operand layout (verified on gfx950): A (16 x 32):
// lane l holds row l%16, k = 8(l/16)..+7; B (32 x 16): lane l holds column
// l%16, the same k; D (16 x 16): lane l holds column l%16, rows 4(l/16)..+3.
// The contraction index only has to agree between A and B, so over tokens
// (k = j) both operands use the slot map e -> j = j0 + 4g + (e%4) + 16(e/4),
// g = l/16, which is exactly the row set of two stacked C_c B_c^T output
// tiles: the masked products become the B operand of the next MFMA in
// registers, and the X / B operands come from row-major LDS through 16-bit
// transpose reads.
//
// Work split inside the workgroup: output rows (16-token tiles) are dealt to
// the 4 waves in the pairs (w, 7-w, 8+w, 15-w) so every wave gets the same
// number of lower-triangular tiles; state tiles (16 x 16 of N x P) are split
// by n so each wave needs the B_c^T fragments of its own n range only.
#pragma once

#include "ssd_common.hpp"
#include "ssd_segsum.hpp"

namespace ssd {

template <int Q, int N, int PB>
struct Bf16Cfg {
    static constexpr int NT = N / 16;                 // state n-tiles
    static constexpr int PT = PB / 16;                // headdim tiles
    static constexpr int KN = (N >= 32) ? N / 32 : 1; // K=32 steps over n
    static constexpr int IT = Q / 64;                 // output row tiles per wave
    static constexpr int ST = (NT * PT + 3) / 4;      // state tiles per wave
    static constexpr int NTW = (NT >= 4) ? NT / 4 : 1;
    static constexpr int PTW = ST / NTW;
    static constexpr int LDB = N + 8;                 // padded LDS row pitch (elements)
    static constexpr int LDX = PB + 8;
    static constexpr int LDH = N + 8;
    static constexpr size_t kLdsBytes =
        (size_t)(Q * LDB + Q * LDX + PB * LDH) * 2 + sizeof(SegLds<Q>);
    static_assert(Q % 64 == 0 && Q <= 256, "chunk size");
    static_assert(N % 16 == 0 && N <= 128, "dstate");
    static_assert(PB % 16 == 0 && PB <= 128, "headdim block");
    static_assert(ST % NTW == 0, "state tile split");
};

template <int Q, int N, int PB>
__device__ inline int owned_tile(int wave, int k) {
    const int m = k >> 1;
    return (k & 1) ? (8 * m + 7 - wave) : (8 * m + wave);
}

// Eight k-consecutive bf16 at p (16-byte aligned LDS or global), or zeros.
__device__ inline bf16x8 load8(const bf16 *p, bool ok) {
    if (!ok) return bf16x8{};
    return *(const bf16x8 *)p;
}

template <int Q, int N, int PB>
__global__ __launch_bounds__(kThreads, 1) void ssd_chunk_bf16_kernel(ChunkArgs a) {
    using Cfg = Bf16Cfg<Q, N, PB>;
    constexpr int NT = Cfg::NT, PT = Cfg::PT, KN = Cfg::KN, IT = Cfg::IT;
    constexpr int ST = Cfg::ST, NTW = Cfg::NTW, PTW = Cfg::PTW;
    constexpr int LDB = Cfg::LDB, LDX = Cfg::LDX, LDH = Cfg::LDH;
    static_assert(Cfg::kLdsBytes <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) bf16 sB[Q * LDB];
    __shared__ __attribute__((aligned(16))) bf16 sX[Q * LDX];
    __shared__ __attribute__((aligned(16))) bf16 sH[PB * LDH];
    __shared__ __attribute__((aligned(16))) SegLds<Q> sg;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const Unit un = unit_of_block(a);
    const int b = un.b, h = un.h, s = un.s, pb = un.pb;
    // The last split's local summary is never used (its entering state comes
    // from the scan and its end state is the final state).
    if (a.mode == kModeSplitLocal && s == a.nsplits - 1) return;
    const int L = a.seqlen, H = a.nheads, G = a.ngroups, P = a.headdim;
    const int grp = h / (H / G);
    const bool full = a.mode == kModeFull;
    const int c_begin = s * a.split_chunks;
    const int c_end = min(a.nchunks, c_begin + a.split_chunks);

    const bf16 *xg = (const bf16 *)a.x;
    const bf16 *Bg = (const bf16 *)a.B;
    const bf16 *Cg = (const bf16 *)a.C;
    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.f;
    const float *dt_row = a.dt + (int64_t)b * L * H + h;
    const int32_t *seq_row = a.seq_idx ? a.seq_idx + (int64_t)b * L : nullptr;
    const int p_base = pb * PB;

    // State tiles owned by this wave: n-tiles nt0.., headdim tiles pt0..
    const int st_first = wave * ST;
    const bool st_valid = st_first < NT * PT;
    const int nt0 = st_first / PT, pt0 = st_first % PT;

    f32x4 hs[ST];
    {
        const float *src = nullptr;
        if (full && s == 0) src = a.init_states ? a.init_states + ((int64_t)b * H + h) * P * N : nullptr;
        else if (full) src = a.ws_states + (((int64_t)b * H + h) * a.nsplits + s) * P * N;
#pragma unroll
        for (int k = 0; k < ST; ++k) {
            const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (src && st_valid) {
                const int p = p_base + pt * 16 + l16, n = nt * 16 + 4 * g;
                v = *(const f32x4 *)(src + (int64_t)p * N + n);
            }
            hs[k] = v;
        }
        if (full && st_valid) {
#pragma unroll
            for (int k = 0; k < ST; ++k) {
                const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
                *(bf16x4 *)&sH[(pt * 16 + l16) * LDH + nt * 16 + 4 * g] = f32x4_to_bf16x4(hs[k]);
            }
        }
    }
    float split_decay = 1.f;

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * Q;
        const int nvalid = min(Q, L - t0);

        // ---- 1. stage B_c and X_c in LDS, token values of the segsum
        {
            constexpr int BV = N / 8;
            const bf16 *Bsrc = Bg + ((int64_t)b * L * G + grp) * N;
#pragma unroll 4
            for (int v = tid; v < Q * BV; v += kThreads) {
                const int row = v / BV, cv = v % BV;
                bf16x8 val = bf16x8{};
                if (row < nvalid) val = *(const bf16x8 *)(Bsrc + (int64_t)(t0 + row) * G * N + cv * 8);
                *(bf16x8 *)&sB[row * LDB + cv * 8] = val;
            }
            constexpr int XV = PB / 8;
            const bf16 *Xsrc = xg + ((int64_t)b * L * H + h) * P + p_base;
#pragma unroll 4
            for (int v = tid; v < Q * XV; v += kThreads) {
                const int row = v / XV, cv = v % XV;
                bf16x8 val = bf16x8{};
                if (row < nvalid) val = *(const bf16x8 *)(Xsrc + (int64_t)(t0 + row) * H * P + cv * 8);
                *(bf16x8 *)&sX[row * LDX + cv * 8] = val;
            }
        }
        int flag_any = 0;
        if (tid < Q) {
            seg_load_token<Q>(sg, tid, t0, nvalid, dt_row, H, A_h, seq_row);
            flag_any = sg.flag[tid];
        }
        flag_any = __syncthreads_or(flag_any);
        if (tid == 0) sg.any_reset = flag_any;

        // C_c rows of this wave's output tiles, straight to registers.
        bf16x8 cf[IT][KN];
        if (full) {
            const bf16 *Csrc = Cg + ((int64_t)b * L * G + grp) * N;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int i = owned_tile<Q, N, PB>(wave, it) * 16 + l16;
#pragma unroll
                for (int kk = 0; kk < KN; ++kk) {
                    const int col = kk * 32 + 8 * g;
                    cf[it][kk] = load8(Csrc + (int64_t)(t0 + i) * G * N + col,
                                       i < nvalid && col < N);
                }
            }
        }

        // ---- 2./3. segsum factors
        if (tid < Q) seg_block_sums<Q>(sg, tid);
        __syncthreads();
        if (tid < Q) seg_chunk_products<Q>(sg, tid);
        __syncthreads();

        const float Tc = sg.T;
        split_decay = __fmul_rn(split_decay, Tc);
#pragma unroll
        for (int k = 0; k < ST; ++k) hs[k] *= Tc;

        // ---- 4. output: state projection, diagonal block, skip
        f32x4 acc[IT][PT];
        float ediag[IT][4];
        float Fch[IT];
        int rs_i[IT];
        if (full) {
#pragma unroll
            for (int it = 0; it < IT; ++it)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[it][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
            // Y^T += h^T C^T  (A = h^T rows p, B = C rows i; k = n)
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int col = kk * 32 + 8 * g;
                    const bf16x8 hfrag = load8(&sH[(pt * 16 + l16) * LDH + col], col < N);
#pragma unroll
                    for (int it = 0; it < IT; ++it) acc[it][pt] = mfma_bf16(hfrag, cf[it][kk], acc[it][pt]);
                }
            }
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int I = owned_tile<Q, N, PB>(wave, it);
                const int i = I * 16 + l16;
                const float ui = sg.u[i];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[it][pt] *= ui;
                rs_i[it] = sg.rs[i];
                const float sum0 = seg_diag_row(sg.d, I * 16, i, g, ediag[it]);
                Fch[it] = seg_chain_start(sum0, I * 16, rs_i[it]);
            }
        }

        // Token pairs of 16-row tiles, last to first (the F chain runs leftwards).
        for (int m = Q / 32 - 1; m >= 0; --m) {
            const int jr0 = 32 * m + 4 * g;   // rows of slots e = 0..3; +16 for e = 4..7
            // X_c fragments: lane (p = 16 pt + l16) holds X[j][p] at the slot rows.
            bf16x8 xa[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const bf16 *p0 = &sX[(jr0 + (l16 >> 2)) * LDX + pt * 16 + 4 * (l16 & 3)];
                xa[pt] = join_bf16x8(lds_read_tr16(p0), lds_read_tr16(p0 + 16 * LDX));
            }
            // chunk state: h += (B_c^T diag(w dt)) X_c over these 32 tokens
            if (st_valid) {
                const f32x4 w0 = *(const f32x4 *)&sg.wcd[jr0];
                const f32x4 w1 = *(const f32x4 *)&sg.wcd[jr0 + 16];
#pragma unroll
                for (int an = 0; an < NTW; ++an) {
                    const int nt = nt0 + an;
                    const bf16 *p0 = &sB[(jr0 + (l16 >> 2)) * LDB + nt * 16 + 4 * (l16 & 3)];
                    const bf16x8 raw = join_bf16x8(lds_read_tr16(p0), lds_read_tr16(p0 + 16 * LDB));
                    bf16x8 bt;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bt[e] = (bf16)((float)raw[e] * w0[e]);
                        bt[e + 4] = (bf16)((float)raw[e + 4] * w1[e]);
                    }
#pragma unroll
                    for (int bp = 0; bp < PTW; ++bp)
                        hs[an * PTW + bp] = mfma_bf16(bt, xa[pt0 + bp], hs[an * PTW + bp]);
                }
            }
            if (!full) continue;

            // diagonal block: S^T = B_c C_c^T on the two 16-token tiles, masked
            bool need = false;
#pragma unroll
            for (int it = 0; it < IT; ++it) need |= owned_tile<Q, N, PB>(wave, it) >= 2 * m;
            if (!need) continue;
            bf16x8 bfr[2][KN];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int kk = 0; kk < KN; ++kk) {
                    const int col = kk * 32 + 8 * g;
                    bfr[hf][kk] = load8(&sB[(32 * m + 16 * hf + l16) * LDB + col], col < N);
                }
            const f32x4 dt0 = *(const f32x4 *)&sg.dt[jr0];
            const f32x4 dt1 = *(const f32x4 *)&sg.dt[jr0 + 16];
            const f32x4 W0 = *(const f32x4 *)&sg.W[jr0];
            const f32x4 W1 = *(const f32x4 *)&sg.W[jr0 + 16];
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int I = owned_tile<Q, N, PB>(wave, it);
                if (I < 2 * m) continue;
                const int i = I * 16 + l16;
                bf16x8 pf;
#pragma unroll
                for (int hf = 1; hf >= 0; --hf) {
                    const int jt = 2 * m + hf;
                    const f32x4 dtv = hf ? dt1 : dt0;
                    const f32x4 Wv = hf ? W1 : W0;
                    if (jt > I) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) pf[hf * 4 + r] = (bf16)0.f;
                        continue;
                    }
                    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) S = mfma_bf16(bfr[hf][kk], cf[it][kk], S);
                    float Lr[4];
                    if (jt == I) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            Lr[r] = seg_diag_value(ediag[it][r], i, jt * 16 + 4 * g + r, rs_i[it]);
                    } else {
                        if (jt < I - 1) Fch[it] = seg_chain_step(Fch[it], sg.Tb[jt + 1]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) Lr[r] = seg_offdiag(Fch[it], Wv[r]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) pf[hf * 4 + r] = (bf16)(S[r] * Lr[r] * dtv[r]);
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[it][pt] = mfma_bf16(xa[pt], pf, acc[it][pt]);
            }
        }

        if (full) {
            bf16 *yg = (bf16 *)a.y;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int i = owned_tile<Q, N, PB>(wave, it) * 16 + l16;
                if (i >= nvalid) continue;
                bf16 *yrow = yg + (((int64_t)b * L + t0 + i) * H + h) * P + p_base;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int p = pt * 16 + 4 * g;
                    const bf16x4 xv = *(const bf16x4 *)&sX[i * LDX + p];
                    f32x4 o = acc[it][pt];
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] += D_h * (float)xv[r];
                    *(bf16x4 *)(yrow + p) = f32x4_to_bf16x4(o);
                }
            }
        }
        __syncthreads();   // all reads of sB, sX, sH and the segsum values are done
        if (full && st_valid) {
#pragma unroll
            for (int k = 0; k < ST; ++k) {
                const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
                *(bf16x4 *)&sH[(pt * 16 + l16) * LDH + nt * 16 + 4 * g] = f32x4_to_bf16x4(hs[k]);
            }
        }
    }

    // ---- split end: final states (last split) or the split's local summary
    if (!st_valid) return;
    float *dst = nullptr;
    if (full) {
        if (s == a.nsplits - 1 && a.final_states) dst = a.final_states + ((int64_t)b * H + h) * P * N;
    } else {
        dst = a.ws_states + (((int64_t)b * H + h) * a.nsplits + s) * P * N;
        if (tid == 0 && pb == 0) a.ws_decay[((int64_t)b * H + h) * a.nsplits + s] = split_decay;
    }
    if (dst) {
#pragma unroll
        for (int k = 0; k < ST; ++k) {
            const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
            const int p = p_base + pt * 16 + l16, n = nt * 16 + 4 * g;
            *(f32x4 *)(dst + (int64_t)p * N + n) = hs[k];
        }
    }
}

}  // namespace ssd
