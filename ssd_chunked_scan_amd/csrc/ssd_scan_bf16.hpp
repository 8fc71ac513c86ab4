// bf16 head kernel of the SSD forward pass on gfx950 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// One workgroup owns one (batch row, head, sequence split, headdim block)
// and walks the split's chunks in order, carrying the N x P state in fp32
// registers (page "NVIDIA Accelerates Mamba-2 Forward Kernel with CUDA
// Tile", "What CUDA Tile Is": tile by tile with the state kept on chip).
// Per chunk c of Q tokens (page "State Space Duality and Mamba-2", "The SSD
// Block Decomposition Algorithm"):
//
//   output   Y^T = (h_{c-1}^T C_c^T) diag(u)                     state projection
//                + X_c^T ((C_c B_c^T) o L o dt + D I)^T           diagonal block + skip
//   state    h_c = T_c h_{c-1} + B_c^T diag(w dt) X_c             chunk state
//
// C_c B_c^T is head-independent; ssd_cb.hip evaluates it once per group and
// chunk (and B_c token-transposed), in the exact per-lane order in which it is
// loaded here, so the heads only apply their own decay mask.  The skip term
// D x is the diagonal D I added to the intra-chunk matrix: it rides on the
// diagonal-block MFMA.
//
// Everything is computed transposed (rows = headdim p) so that each lane of
// an output tile owns one token i and four consecutive p: the row scale u_i
// is one value per lane and y is written 8 bytes per lane.
//
// MFMA 16x16x32 bf16 operand layout (verified on gfx950): A (16 x 32):
// lane l holds row l%16, k = 8(l/16)..+7; B (32 x 16): lane l holds column
// l%16, the same k; D (16 x 16): lane l holds column l%16, rows 4(l/16)..+3.
// Over tokens (k = j) both operands use the slot map
// e -> j = j0 + 4g + (e%4) + 16(e/4), g = l/16: the X operand comes from
// row-major LDS through 16-bit transpose reads, the masked C B^T blocks and
// B^T come from the per-group buffers in that order.
//
// Work split inside the workgroup: W waves (8 for Q = 256, else 4).  Output
// rows (16-token tiles) are dealt in the pairs (w, Q/16-1-w) so every wave
// gets the same number of lower-triangular tiles; state tiles (16 x 16 of
// N x P) are split by n first.
//
// Pipelining, one barrier per chunk: X_{c+1} reaches LDS through asynchronous
// direct loads (global_load_lds_dwordx4) issued at the start of chunk c into
// the other half of a double buffer; the h tile (bf16, operand of the state
// projection) and the segsum values are double-buffered too and written for
// chunk c+1 at the end of chunk c.  C_{c+1} rows go to registers during chunk
// c, the C B^T and B^T fragments two 32-token pairs ahead, and y of chunk c
// is stored at the start of chunk c+1, so the wait before the barrier never
// waits for fresh stores.
#pragma once

#include "ssd_common.hpp"
#include "ssd_segsum.hpp"
#include "ssd_tiles.hpp"

namespace ssd {

template <int Q, int N, int PB>
struct ScanCfg {
    static constexpr int W = (Q == 256) ? 8 : 4;        // waves per workgroup
    static constexpr int THREADS = 64 * W;
    static constexpr int NT = N / 16;                    // state n-tiles
    static constexpr int PT = PB / 16;                   // headdim tiles
    static constexpr int KN = (N >= 32) ? N / 32 : 1;    // K=32 steps over n
    static constexpr int TILES = Q / 16;                 // 16-token row tiles
    static constexpr int NP = Q / 32;                    // 32-token column pairs
    static constexpr int NB = Q / 16;                    // segsum sub-blocks
    static constexpr int IT = (TILES >= 2 * W) ? 2 : 1;  // row tiles per wave
    static constexpr int ST = (NT * PT + W - 1) / W;     // state tiles per wave
    static constexpr int NTW = (NT >= W) ? NT / W : 1;   // n-tiles per wave
    static constexpr int PTW = ST / NTW;                 // headdim tiles per n-tile
    static constexpr bool kAllP = (PTW == PT);           // a wave's state tiles span all of P
    static constexpr int CPRX = PB / 8;                  // 16-byte chunks per X_c row
    static constexpr int SX = Q * PB;                    // swizzled, unpadded X tile
    static constexpr int LDH = N + 8;                    // padded pitch of the h^T tile
    static constexpr int NBLK = CbShape<Q>::NBLK;
    static constexpr size_t kLdsBytes =
        2 * (size_t)SX * 2 + 2 * (size_t)PB * LDH * 2 + 2 * sizeof(SegBuf<Q>);
    static_assert(Q % 64 == 0 && Q <= 256, "chunk size");
    static_assert(N % 16 == 0 && N <= 128, "dstate");
    static_assert(PB % 16 == 0 && PB <= 128, "headdim block");
    static_assert(ST % NTW == 0, "state tile split");
    static_assert(IT == 1 || TILES == 2 * W, "row tile pairs");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

template <int Q, int N, int PB>
__global__ __launch_bounds__(64 * ((Q == 256) ? 8 : 4)) void ssd_scan_bf16_kernel(ChunkArgs a) {
    using Cfg = ScanCfg<Q, N, PB>;
    constexpr int W = Cfg::W, THREADS = Cfg::THREADS;
    constexpr int NT = Cfg::NT, PT = Cfg::PT, KN = Cfg::KN, IT = Cfg::IT, NP = Cfg::NP;
    constexpr int NB = Cfg::NB, ST = Cfg::ST, NTW = Cfg::NTW, PTW = Cfg::PTW;
    constexpr int CPRX = Cfg::CPRX, LDH = Cfg::LDH, NBLK = Cfg::NBLK;
    static_assert(THREADS == 64 * ((Q == 256) ? 8 : 4), "launch bounds");

    __shared__ __attribute__((aligned(1024))) bf16 sXbuf[2 * Cfg::SX];
    __shared__ __attribute__((aligned(16))) bf16 sHbuf[2 * PB * LDH];
    __shared__ __attribute__((aligned(16))) SegBuf<Q> segbuf[2];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const Unit un = unit_of_block(a);
    const int b = un.b, h = un.h, s = un.s, pb = un.pb;
    // The last split's local summary is never used (its entering state comes
    // from the scan and its end state is the final state).
    if (a.mode == kModeSplitLocal && s == a.nsplits - 1) return;
    const int L = a.seqlen, H = a.nheads, G = a.ngroups, P = a.headdim;
    const int grp = h / (H / G);
    const bool full = a.mode == kModeFull;
    const bool resets = a.seq_idx != nullptr;
    const int c_begin = s * a.split_chunks;
    const int c_end = min(a.nchunks, c_begin + a.split_chunks);

    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.f;
    const float *dt_row = a.dt + (int64_t)b * L * H + h;
    const int32_t *seq_row = resets ? a.seq_idx + (int64_t)b * L : nullptr;
    const int p_base = pb * PB;
    const bf16 *Csrc = (const bf16 *)a.C + ((int64_t)b * L * G + grp) * N;
    const bf16 *Xsrc = (const bf16 *)a.x + ((int64_t)b * L * H + h) * P + p_base;
    const int64_t bg = (int64_t)b * G + grp;
    const bf16x8 *Sws = (const bf16x8 *)a.ws_S + bg * a.nchunks * NBLK * 64;
    const bf16x8 *BTws = (const bf16x8 *)a.ws_BT + bg * a.nchunks * NP * N * 4;

    // Row tiles of this wave (uniform).
    int Irow[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) Irow[it] = row_tile<Cfg>(wave, it);

    // State tiles owned by this wave: n-tiles nt0.., headdim tiles pt0..
    const int st_first = wave * ST;
    const bool st_valid = st_first < NT * PT;
    const int nt0 = st_first / PT, pt0 = st_first % PT;

    f32x4 hs[ST];
    bool state_zero = true;   // uniform: the carried state is known to be 0
    {
        const float *src = nullptr;
        if (full && s == 0) src = a.init_states ? a.init_states + ((int64_t)b * H + h) * P * N : nullptr;
        else if (full) src = a.ws_states + (((int64_t)b * H + h) * a.nsplits + s) * P * N;
        state_zero = src == nullptr;
#pragma unroll
        for (int k = 0; k < ST; ++k) {
            const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (src && st_valid) {
                // h^T tile: lane holds h[p = 16 pt + l16][n = 16 nt + 4g .. +3]
                const int p = p_base + pt * 16 + l16, n = nt * 16 + 4 * g;
                v = *(const f32x4 *)(src + (int64_t)p * N + n);
            }
            hs[k] = v;
        }
    }
    float split_decay = 1.f;

    auto write_h = [&](int buf) {
        if (!full || !st_valid) return;
        bf16 *sH = sHbuf + buf * PB * LDH;
#pragma unroll
        for (int k = 0; k < ST; ++k) {
            const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
            *(bf16x4 *)&sH[(pt * 16 + l16) * LDH + nt * 16 + 4 * g] = f32x4_to_bf16x4(hs[k]);
        }
    };
    auto stage_x = [&](int c) {
        const int t0 = c * Q;
        stage_rows_async<Q, W, CPRX>(sXbuf + (c & 1) * Cfg::SX, Xsrc + (int64_t)t0 * H * P,
                                     (int64_t)H * P, min(Q, L - t0), wave, lane, tid);
    };
    // C_c rows of this wave's row tiles (B operand of the state projection, k = n)
    bf16x8 cf[IT][KN];
    auto load_c = [&](int c) {
        const int t0 = c * Q;
        const int nvalid = min(Q, L - t0);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = Irow[it] * 16 + l16;
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
                const int col = kk * 32 + 8 * g;
                cf[it][kk] = load8(Csrc + (int64_t)(t0 + i) * G * N + col, i < nvalid && col < N);
            }
        }
    };
    float p_dt = 0.f;
    int p_flag = 0;
    auto fetch_token = [&](int c) {
        const int t0 = c * Q;
        if (tid < Q) seg_fetch_token(tid, t0, min(Q, L - t0), dt_row, H, seq_row, p_dt, p_flag);
    };

    // Output tile accumulators: acc[it][pt] = Y^T tile (rows p, columns i).
    f32x4 acc[IT][PT];
    auto store_y = [&](int c) {
        const int t0 = c * Q;
        const int nvalid = min(Q, L - t0);
#pragma unroll
        for (int it = 0; it < IT; ++it) mfma_fence_all(acc[it]);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = Irow[it] * 16 + l16;
            if (i >= nvalid) continue;
            bf16 *yrow = (bf16 *)a.y + (((int64_t)b * L + t0 + i) * H + h) * P + p_base;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                *(bf16x4 *)(yrow + pt * 16 + 4 * g) = f32x4_to_bf16x4(acc[it][pt]);
        }
    };

    if (c_begin < c_end) {
        write_h(c_begin & 1);
        stage_x(c_begin);
        fetch_token(c_begin);
        if (tid < Q) seg_tokens<Q>(segbuf[c_begin & 1], tid, p_dt, p_flag, A_h, resets);
        if (full) load_c(c_begin);
        vmem_lds_sync();
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int buf = c & 1;
        const int t0 = c * Q;
        const bf16 *sX = sXbuf + buf * Cfg::SX;
        const bf16 *sH = sHbuf + buf * PB * LDH;
        const SegBuf<Q> &sg = segbuf[buf];

        // ---- 1. y of the previous chunk; next chunk's X tile and token values
        if (full && c > c_begin) store_y(c - 1);
        if (c + 1 < c_end) {
            stage_x(c + 1);
            fetch_token(c + 1);
        }

        // ---- 2. cross-sub-block decay products; carry the state
        SegProducts<NB> pr;
        seg_products<Q>(sg, pr);
        split_decay = __fmul_rn(split_decay, pr.T);
#pragma unroll
        for (int k = 0; k < ST; ++k) hs[k] *= pr.T;

        // ---- 3. per-row factors of this wave's row tiles
        //   u_i            decay from the previous chunk's state to token i
        //   Fc             the off-diagonal chain F(i, J), started at J = I-1
        //   fdg, dadd      diagonal-sub-block factor L_ij dt_j and the skip D_h
        float u[IT], Fc[IT], fdg[IT][4], dadd[IT][4];
        if (full) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int I = Irow[it], I0 = I * 16, i = I0 + l16;
                const int rs = resets ? seg_last_reset<Q>(sg, i, I) : -1;
                float ev[4];
                const float sum0 = seg_diag_row(sg.d, I0, i, g, ev);
                const float F0 = seg_chain_start(sum0, I0, rs);
                float V = 1.f;
                for (int k = 0; k < I; ++k) V = __fmul_rn(V, sg.Tb[k]);
                u[it] = __fmul_rn(F0, V);
                Fc[it] = F0;
                const f32x4 dtj = *(const f32x4 *)&sg.dt[I0 + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = I0 + 4 * g + r;
                    fdg[it][r] = __fmul_rn(seg_diag_value(ev[r], i, j, rs), dtj[r]);
                    dadd[it][r] = (j == i) ? D_h : 0.f;
                }
            }
        }

        // ---- 4. state projection Y^T = h^T C^T, then the row scale u
        if (full) {
            if (state_zero) {
#pragma unroll
                for (int it = 0; it < IT; ++it)
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[it][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) {
                        const int col = kk * 32 + 8 * g;
                        const bf16x8 hfrag = load8(&sH[(pt * 16 + l16) * LDH + col], col < N);
#pragma unroll
                        for (int it = 0; it < IT; ++it)
                            acc[it][pt] = kk == 0 ? mfma_bf16_zero_acc(hfrag, cf[it][0])
                                                  : mfma_bf16(hfrag, cf[it][kk], acc[it][pt]);
                    }
                }
#pragma unroll
                for (int it = 0; it < IT; ++it) mfma_fence_all(acc[it]);
#pragma unroll
                for (int it = 0; it < IT; ++it)
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[it][pt] *= u[it];
            }
            if (c + 1 < c_end) load_c(c + 1);
        }
        state_zero = false;

        // ---- 5. 32-token column pairs, last to first (the F chain runs leftwards)
        const bf16x8 *Sc = Sws + (int64_t)c * NBLK * 64 + lane;
        const bf16x8 *BTc = BTws + (int64_t)c * NP * N * 4;
        bf16x8 sfr[3][IT], bfr[3][NTW];
        auto load_pair = [&](int m) {
            const int slot = m % 3;
            if (full) {
#pragma unroll
                for (int it = 0; it < IT; ++it)
                    if (2 * m <= Irow[it]) sfr[slot][it] = Sc[(CbShape<Q>::off(Irow[it]) + m) * 64];
            }
            if (st_valid) {
#pragma unroll
                for (int q = 0; q < NTW; ++q)
                    bfr[slot][q] = BTc[((int64_t)m * N + (nt0 + q) * 16 + l16) * 4 + g];
            }
        };
        load_pair(NP - 1);
        if (NP >= 2) load_pair(NP - 2);
#pragma unroll
        for (int m = NP - 1; m >= 0; --m) {
            if (m >= 2) load_pair(m - 2);
            const int slot = m % 3;
            const int jr0 = 32 * m + 4 * g;   // tokens of slots e = 0..3; +16 for e = 4..7
            // X_c fragments: lane (p = 16 pt + l16) holds X[j][p] at the slot tokens.
            bf16x8 xa[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int rr = jr0 + (l16 >> 2), col = pt * 16 + 4 * (l16 & 3);
                xa[pt] = join_bf16x8(lds_read_tr16(&sX[tile_off_col<CPRX>(rr, col)]),
                                     lds_read_tr16(&sX[tile_off_col<CPRX>(rr + 16, col)]));
            }
            const f32x4 wlo = *(const f32x4 *)&sg.wd[jr0];
            const f32x4 whi = *(const f32x4 *)&sg.wd[jr0 + 16];

            // chunk state: h^T += (B_c^T diag(w dt)) X_c over these 32 tokens,
            // w dt = (W dt) Z_J with Z_J the decay after sub-block J
            if (st_valid) {
                f32x4 flo, fhi;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    flo[r] = __fmul_rn(wlo[r], pr.Z[2 * m]);
                    fhi[r] = __fmul_rn(whi[r], pr.Z[2 * m + 1]);
                }
                bf16x8 xs[PTW];
                if constexpr (Cfg::kAllP) {
#pragma unroll
                    for (int k = 0; k < PTW; ++k) xs[k] = xa[k];
                } else {
#pragma unroll
                    for (int k = 0; k < PTW; ++k) {
                        const int rr = jr0 + (l16 >> 2), col = (pt0 + k) * 16 + 4 * (l16 & 3);
                        xs[k] = join_bf16x8(lds_read_tr16(&sX[tile_off_col<CPRX>(rr, col)]),
                                            lds_read_tr16(&sX[tile_off_col<CPRX>(rr + 16, col)]));
                    }
                }
#pragma unroll
                for (int q = 0; q < NTW; ++q) {
                    const bf16x8 bv = bfr[slot][q];
                    bf16x8 bs;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        bs[r] = (bf16)((float)bv[r] * flo[r]);
                        bs[4 + r] = (bf16)((float)bv[4 + r] * fhi[r]);
                    }
#pragma unroll
                    for (int k = 0; k < PTW; ++k)
                        hs[q * PTW + k] = mfma_bf16(bs, xs[k], hs[q * PTW + k]);
                }
            }

            // diagonal block: Y^T += X_c^T (masked C B^T)^T for row tiles I >= 2m
            if (full) {
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int I = Irow[it];
                    if (2 * m > I) continue;
                    const bf16x8 sv = sfr[slot][it];
                    bf16x8 pf;
                    if (m == (I >> 1)) {
                        if (I & 1) {
                            // slots 0..3: sub-block I-1 (chain start); 4..7: diagonal
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                pf[r] = (bf16)((float)sv[r] * __fmul_rn(Fc[it], wlo[r]));
                                pf[4 + r] = (bf16)fmaf((float)sv[4 + r], fdg[it][r], dadd[it][r]);
                            }
                            Fc[it] = __fmul_rn(Fc[it], pr.Tb[2 * m]);
                        } else {
                            // slots 0..3: diagonal; 4..7: above the diagonal
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                pf[r] = (bf16)fmaf((float)sv[r], fdg[it][r], dadd[it][r]);
                                pf[4 + r] = (bf16)0.f;
                            }
                        }
                    } else {
                        // both sub-blocks left of the diagonal: Fc = F(i, 2m+1)
                        const float Flo = __fmul_rn(Fc[it], pr.Tb[2 * m + 1]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            pf[4 + r] = (bf16)((float)sv[4 + r] * __fmul_rn(Fc[it], whi[r]));
                            pf[r] = (bf16)((float)sv[r] * __fmul_rn(Flo, wlo[r]));
                        }
                        Fc[it] = __fmul_rn(Flo, pr.Tb[2 * m]);
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[it][pt] = mfma_bf16(xa[pt], pf, acc[it][pt]);
                }
            }
        }

        // ---- 6. hand the next chunk its h tile and segsum values
        if (c + 1 < c_end) {
            mfma_fence_all(hs);
            write_h((c + 1) & 1);
            if (tid < Q) seg_tokens<Q>(segbuf[(c + 1) & 1], tid, p_dt, p_flag, A_h, resets);
            vmem_lds_sync();   // X_{c+1} has landed; all reads of this chunk's buffers are done
        }
    }
    if (full && c_begin < c_end) store_y(c_end - 1);

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
        mfma_fence_all(hs);
#pragma unroll
        for (int k = 0; k < ST; ++k) {
            const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
            const int p = p_base + pt * 16 + l16, n = nt * 16 + 4 * g;
            *(f32x4 *)(dst + (int64_t)p * N + n) = hs[k];
        }
    }
}

}  // namespace ssd
