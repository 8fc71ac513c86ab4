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
// chunk c+1 at the end of chunk c.  The C rows of chunk c+1 go to registers
// last in chunk c and stay in flight across the barrier (its wait counts them
// out), the C B^T and B^T fragments one 32-token pair ahead of their use, and
// y of chunk c is stored at the start of chunk c+1, so the wait before the
// barrier never waits for fresh stores.
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
        2 * (size_t)SX * 2 + 2 * (size_t)PB * LDH * 2 + 2 * sizeof(SegBuf<Q>);   // X stage + work
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

    // X tiles: the asynchronous loads land in sXstage (written only by them)
    // and are copied to sXwork (read only by the MFMA operand reads) after the
    // chunk's barrier.  Two distinct LDS objects let the compiler see that
    // reads of the current tile do not wait for the loads in flight.
    __shared__ __attribute__((aligned(1024))) bf16 sXstage[Cfg::SX];
    __shared__ __attribute__((aligned(1024))) bf16 sXwork[Cfg::SX];
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
    if (c_begin >= c_end) return;

    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.f;
    const float *dt_row = a.dt + (int64_t)b * L * H + h;
    // Without seq_idx the document-id loads read dt bits of the same row
    // instead (any valid address; the values are not used).
    const int32_t *seq_row = resets ? a.seq_idx + (int64_t)b * L : (const int32_t *)(a.dt + (int64_t)b * L * H);
    const int p_base = pb * PB;
    const bf16 *Csrc = (const bf16 *)a.C + ((int64_t)b * L * G + grp) * N;
    const bf16 *Xsrc = (const bf16 *)a.x + ((int64_t)b * L * H + h) * P + p_base;
    const int64_t bg = (int64_t)b * G + grp;
    const bf16x8 *Sws = (const bf16x8 *)a.ws_S + bg * a.nchunks * NBLK * 64 + lane;
    const bf16x8 *BTws = (const bf16x8 *)a.ws_BT + bg * a.nchunks * NP * N * 4;

    // Row tiles of this wave: I0 = w < TILES/2 and, with two per wave,
    // I1 = TILES-1-w >= TILES/2.  So for pairs m >= NP/2 only I1 can reach
    // the pair, and for m < NP/2 the pair lies wholly left of I1's diagonal.
    int Irow0[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) Irow0[it] = row_tile<Cfg>(wave, it);

    // State tiles owned by this wave: n-tiles nt0.., headdim tiles pt0..
    const int st_first = wave * ST;
    const bool st_valid = st_first < NT * PT;
    const int nt0 = st_valid ? st_first / PT : 0, pt0 = st_valid ? st_first % PT : 0;

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
    // X rows of chunk c into sXstage (asynchronous)
    auto stage_x = [&](int c) {
        const int t0 = c * Q;
        stage_rows_async<Q, W, CPRX>(sXstage, Xsrc + (int64_t)t0 * H * P, (int64_t)H * P,
                                     min(Q, L - t0), wave, lane);
    };
    // sXstage -> sXwork, 16 bytes per thread and step (between two barriers)
    auto copy_x = [&]() {
#pragma unroll
        for (int k = 0; k < (Cfg::SX + 8 * THREADS - 1) / (8 * THREADS); ++k) {
            const int e = (k * THREADS + tid) * 8;
            if (Cfg::SX % (8 * THREADS) == 0 || e < Cfg::SX)
                *(bf16x8 *)&sXwork[e] = *(const bf16x8 *)&sXstage[e];
        }
    };
    // C_c rows of this wave's row tiles (B operand of the state projection,
    // k = n); rows past the end of the sequence read row L-1 (their outputs
    // are not stored), columns past dstate are zeroed at use.
    bf16x8 cf[IT][KN];
    auto load_c = [&](int c, const int (&Irow)[IT]) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int t = min(c * Q + Irow[it] * 16 + l16, L - 1);
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
                const int col = min(kk * 32 + 8 * g, N - 8);
                cf[it][kk] = *(const bf16x8 *)(Csrc + (int64_t)t * G * N + col);
            }
        }
    };
    // Raw token values of a chunk for thread tid % Q (selected at use).
    float p_dt = 0.f;
    int p_cur = 0, p_prev = 0;
    auto fetch_token = [&](int c) {
        const int tg = min(c * Q + tid % Q, L - 1);
        p_dt = dt_row[(int64_t)tg * H];
        p_cur = seq_row[tg];
        p_prev = seq_row[max(tg - 1, 0)];
    };
    auto tokens = [&](int c, int buf) {
        if (tid < Q) {
            const int tg = c * Q + tid;
            const bool valid = tg < L;
            const float dtv = valid ? p_dt : 0.f;
            const int flag = (resets && valid && tg > 0 && p_cur != p_prev) ? 1 : 0;
            seg_tokens<Q>(segbuf[buf], tid, dtv, flag, A_h, resets);
        }
    };

    // Output tile accumulators: acc[it][pt] = Y^T tile (rows p, columns i).
    f32x4 acc[IT][PT];
    auto store_y = [&](int c, const int (&Irow)[IT]) {
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

    // ---- prologue: state tile, X, token values and C rows of the first chunk
    write_h(c_begin & 1);
    stage_x(c_begin);
    fetch_token(c_begin);
    tokens(c_begin, c_begin & 1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    load_c(c_begin, Irow0);
    vmem_lds_sync_keep<IT * KN>();   // the C rows may still be in flight
    copy_x();
    lds_sync();

    for (int c = c_begin; c < c_end; ++c) {
        // The row tiles pass through an empty asm once per chunk, so that
        // the compiler recomputes the few scalar values derived from them
        // here instead of keeping dozens of them live across the loop.
        int Irow[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            Irow[it] = Irow0[it];
            asm volatile("" : "+s"(Irow[it]));
        }
        const int buf = c & 1;
        const bf16 *sX = sXwork;
        const bf16 *sH = sHbuf + buf * PB * LDH;
        const SegBuf<Q> &sg = segbuf[buf];
        const int cn = min(c + 1, c_end - 1);   // next chunk (the last one repeats itself)

        // ---- 1. loads, in this order: this chunk's C rows and the first
        // column pair's fragments, the next chunk's X tile, y of the previous
        // chunk and the next token values.  Vector-memory completions are
        // counted in issue order, so waiting for the C rows or the first
        // fragments does not wait for the X tile.
        const bf16x8 *Sc = Sws + (int64_t)c * NBLK * 64;
        const bf16x8 *BTc = BTws + (int64_t)c * NP * N * 4;
        bf16x8 sfr[2][IT], bfr[2][NTW];
        // Fragments of pair m, loaded unconditionally (a row tile that does not
        // reach the pair loads its own diagonal block instead, unused).
        auto load_pair = [&](int m) {
            const int slot = m & 1;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                if (IT == 2 && it == 0 && m >= NP / 2) continue;   // never reaches the pair
                const int I = Irow[it];
                sfr[slot][it] = Sc[(CbShape<Q>::off(I) + min(m, I >> 1)) * 64];
            }
#pragma unroll
            for (int q = 0; q < NTW; ++q)
                bfr[slot][q] = BTc[((int64_t)m * N + min(nt0 + q, NT - 1) * 16 + l16) * 4 + g];
        };
        load_pair(NP - 1);
        stage_x(cn);
        if (full && c > c_begin) store_y(c - 1, Irow);
        fetch_token(cn);

        // ---- 2. cross-sub-block decay products V_I (this wave's row tiles)
        // and T; carry the state
        float VI[IT], T;
        {
            float Tb[NB];
#pragma unroll
            for (int k = 0; k < NB; k += 4) {
                const f32x4 v = *(const f32x4 *)&sg.Tb[k];
#pragma unroll
                for (int r = 0; r < 4; ++r) Tb[k + r] = v[r];
            }
            seg_prefix_products<NB, IT>(Tb, Irow, VI, T);
        }
        split_decay = __fmul_rn(split_decay, T);
#pragma unroll
        for (int k = 0; k < ST; ++k) hs[k] *= T;

        // ---- 3. per-row factors of this wave's row tiles
        //   u_i            decay from the previous chunk's state to token i
        //   Fc             the off-diagonal chain F(i, J), started at J = I-1
        //   fdg            diagonal-sub-block factor L_ij dt_j
        float u[IT], Fc[IT], fdg[IT][4];
        if (full) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int I = Irow[it], I0 = I * 16, i = I0 + l16;
                const int rs = resets ? seg_last_reset<Q>(sg, i, I) : -1;
                float dd[16];
#pragma unroll
                for (int k = 0; k < 16; k += 4) {
                    const f32x4 v = *(const f32x4 *)&sg.d[I0 + k];
#pragma unroll
                    for (int r = 0; r < 4; ++r) dd[k + r] = v[r];
                }
                float ev[4];
                const float sum0 = seg_diag_row_regs(dd, I0, i, g, ev);
                const float F0 = seg_chain_start(sum0, I0, rs);
                u[it] = __fmul_rn(F0, VI[it]);
                Fc[it] = F0;
                const f32x4 dtj = *(const f32x4 *)&sg.dt[I0 + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = I0 + 4 * g + r;
                    fdg[it][r] = __fmul_rn(seg_diag_value(ev[r], i, j, rs), dtj[r]);
                }
            }
        }

        // ---- 4. state projection Y^T = h^T C^T, then the row scale u
        if (full) {
            if constexpr (N < 32) {
                // k = n runs over 32 columns; zero the ones past dstate
#pragma unroll
                for (int it = 0; it < IT; ++it)
                    if (8 * g >= N) cf[it][0] = bf16x8{};
            }
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
                        const int col = min(kk * 32 + 8 * g, N - 8);
                        bf16x8 hfrag = *(const bf16x8 *)&sH[(pt * 16 + l16) * LDH + col];
                        if constexpr (N < 32) {
                            if (8 * g >= N) hfrag = bf16x8{};
                        }
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
        }
        state_zero = false;

        // ---- 5. 32-token column pairs, last to first (the F chain runs leftwards)
        float Zrun = 1.f;   // decay from the end of sub-block 2m+1 to the chunk end
#pragma unroll
        for (int m = NP - 1; m >= 0; --m) {
            if (m >= 1) load_pair(m - 1);
            const int slot = m & 1;
            // consume the pair's fragments here on every path, so that their
            // loads stay where they were issued
#pragma unroll
            for (int it = 0; it < IT; ++it)
                if (!(IT == 2 && it == 0 && m >= NP / 2)) asm volatile("" ::"v"(sfr[slot][it]));
            const int jr0 = 32 * m + 4 * g;   // tokens of slots e = 0..3; +16 for e = 4..7
            // whole-sub-block decays of the pair and the suffix products Z
            // (Z_J = Z_{J+1} Tb_{J+1}, as in seg_chunk_products)
            const float Tb_lo = sg.Tb[2 * m], Tb_hi = sg.Tb[2 * m + 1];
            const float Z_hi = Zrun, Z_lo = __fmul_rn(Zrun, Tb_hi);
            Zrun = __fmul_rn(Z_lo, Tb_lo);
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
                    flo[r] = __fmul_rn(wlo[r], Z_lo);
                    fhi[r] = __fmul_rn(whi[r], Z_hi);
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
                    // statically known: with two row tiles per wave, tile 0
                    // never reaches the upper half of the pairs and tile 1 lies
                    // wholly right of the lower half
                    if (IT == 2 && it == 0 && m >= NP / 2) continue;
                    const bool whole = (IT == 2 && it == 1 && m < NP / 2) || m < (I >> 1);
                    if (!whole && m > (I >> 1)) continue;
                    const bf16x8 sv = sfr[slot][it];
                    bf16x8 pf;
                    if (whole) {
                        // both sub-blocks left of the diagonal: Fc = F(i, 2m+1)
                        const float Flo = __fmul_rn(Fc[it], Tb_hi);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            pf[4 + r] = (bf16)((float)sv[4 + r] * __fmul_rn(Fc[it], whi[r]));
                            pf[r] = (bf16)((float)sv[r] * __fmul_rn(Flo, wlo[r]));
                        }
                        Fc[it] = __fmul_rn(Flo, Tb_lo);
                    } else if (I & 1) {
                        // slots 0..3: sub-block I-1 (chain start); 4..7: diagonal
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            pf[r] = (bf16)((float)sv[r] * __fmul_rn(Fc[it], wlo[r]));
                            pf[4 + r] = (bf16)fmaf((float)sv[4 + r], fdg[it][r],
                                                   (4 * g + r == l16) ? D_h : 0.f);
                        }
                        Fc[it] = __fmul_rn(Fc[it], Tb_lo);
                    } else {
                        // slots 0..3: diagonal; 4..7: above the diagonal
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            pf[r] = (bf16)fmaf((float)sv[r], fdg[it][r], (4 * g + r == l16) ? D_h : 0.f);
                            pf[4 + r] = (bf16)0.f;
                        }
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[it][pt] = mfma_bf16(xa[pt], pf, acc[it][pt]);
                }
            }
        }

        // ---- 6. hand the next chunk its h tile and segsum values (also after
        // the last chunk, harmlessly: an unconditional wait here lets the
        // compiler see that nothing is in flight at the top of the loop)
        mfma_fence_all(hs);
        write_h(buf ^ 1);
        tokens(c + 1, buf ^ 1);
        // the next chunk's C rows go out last: the barrier lets them stay in
        // flight, while X_{c+1} (issued earlier) has landed and every read of
        // this chunk's buffers is done
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        load_c(cn, Irow);
        vmem_lds_sync_keep<IT * KN>();
        copy_x();
        lds_sync();
    }
    if (full) store_y(c_end - 1, Irow0);

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
