// bf16 chunk kernel of the SSD forward pass on gfx950 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// One workgroup owns one (batch row, head, sequence split, headdim block)
// and walks the split's chunks in order, carrying the N x P state in fp32
// registers (page "NVIDIA Accelerates Mamba-2 Forward Kernel with CUDA
// Tile", "What CUDA Tile Is": tile by tile with the state kept on chip).  Per
// chunk c of Q tokens (page "State Space Duality and Mamba-2", "The SSD
// Block Decomposition Algorithm"):
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
// Work split inside the workgroup: W waves (8 for Q = 256, else 4).  Output
// rows (16-token tiles) are dealt in the pairs (w, Q/16-1-w) so every wave
// gets the same number of lower-triangular tiles; state tiles (16 x 16 of
// N x P) are split by n so each wave needs the B_c^T fragments of its own n
// range only.
//
// Pipelining: X_c and B_c reach LDS through asynchronous direct loads
// (global_load_lds_dwordx4: lane l writes 16 bytes at the wave's LDS base +
// 16 l, from any global address).  X is double-buffered and fetched one chunk
// ahead; B is refilled as soon as the previous chunk is done with it and
// lands while the segsum of the next chunk runs.  The wave's C_c rows and the
// token values go to registers one chunk ahead.  Barriers order LDS traffic
// only; the direct loads are waited for explicitly before their first use.
#pragma once

#include "ssd_common.hpp"
#include "ssd_segsum.hpp"

namespace ssd {

template <int Q, int N, int PB>
struct Bf16Cfg {
    static constexpr int W = (Q == 256) ? 8 : 4;        // waves per workgroup
    static constexpr int THREADS = 64 * W;
    static constexpr int NT = N / 16;                    // state n-tiles
    static constexpr int PT = PB / 16;                   // headdim tiles
    static constexpr int KN = (N >= 32) ? N / 32 : 1;    // K=32 steps over n
    static constexpr int TILES = Q / 16;                 // 16-token row tiles
    static constexpr int IT = (TILES >= 2 * W) ? 2 : 1;  // row tiles per wave
    static constexpr int ST = (NT * PT + W - 1) / W;     // state tiles per wave
    static constexpr int NTW = (NT >= W) ? NT / W : 1;   // n-tiles per wave
    static constexpr int PTW = ST / NTW;                 // headdim tiles per n-tile
    static constexpr int CPRB = N / 8;                   // 16-byte chunks per B_c row
    static constexpr int CPRX = PB / 8;                  // 16-byte chunks per X_c row
    static constexpr int SB = Q * N;                     // swizzled, unpadded tiles
    static constexpr int SX = Q * PB;
    static constexpr int LDH = N + 8;                    // padded pitch of the h^T tile
    static constexpr size_t kFixedBytes = (size_t)(SB + PB * LDH) * 2 + sizeof(SegLds<Q>) + 64;
    // X_c double-buffered (fetched a whole chunk ahead) when it fits.
    static constexpr int XBUF = (kFixedBytes + 2 * (size_t)SX * 2 <= 160 * 1024) ? 2 : 1;
    static constexpr size_t kLdsBytes = kFixedBytes + (size_t)XBUF * SX * 2;
    static_assert(Q % 64 == 0 && Q <= 256, "chunk size");
    static_assert(N % 16 == 0 && N <= 128, "dstate");
    static_assert(PB % 16 == 0 && PB <= 128, "headdim block");
    static_assert(ST % NTW == 0, "state tile split");
    static_assert(IT == 1 || TILES == 2 * W, "row tile pairs");
};

// Row tile k of wave w: the pair (w, TILES-1-w), or tile w alone.
template <class Cfg>
__device__ inline int row_tile(int w, int k) {
    return (Cfg::IT == 2 && k == 1) ? (Cfg::TILES - 1 - w) : w;
}

// Swizzled LDS tiles: row r of a tile with CPR 16-byte chunks per row starts at
// element r * CPR * 8 and holds logical chunk c at physical chunk c ^ swz(r).
// With R = 16 / CPR rows per 256 bytes (one pass over the banks) and
// q = r / R, swz = 2q mod CPR + (q / (CPR/2)) mod 2: 16 consecutive rows read
// at one logical chunk (16-byte reads) land in 16 different bank groups, and
// the 4 consecutive rows x 2 chunks of a transpose read do not collide.
template <int CPR>
__device__ inline int swz(int r) {
    constexpr int R = 16 / CPR;
    const int q = r / R;
    return ((2 * q) % CPR + (q / (CPR / 2)) % 2) & (CPR - 1);
}

template <int CPR>
__device__ inline int tile_off(int r, int c) {
    return r * (CPR * 8) + ((c ^ swz<CPR>(r)) << 3);
}

// Element offset of column col (a multiple of 4) of row r in a swizzled tile.
template <int CPR>
__device__ inline int tile_off_col(int r, int col) {
    return tile_off<CPR>(r, col >> 3) + (col & 7);
}

// Eight k-consecutive bf16 at p (16-byte aligned LDS or global), or zeros.
__device__ inline bf16x8 load8(const bf16 *p, bool ok) {
    if (!ok) return bf16x8{};
    return *(const bf16x8 *)p;
}

// Workgroup barrier ordering LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (the prefetch).
__device__ inline void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Barrier after which every direct-to-LDS load issued before it has landed.
__device__ inline void vmem_lds_sync() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Asynchronously copy rows [0, nvalid) of a Q-row tile (CPR 16-byte chunks
// per row, row r at src + r * gstride elements) into a swizzled LDS tile; rows
// [nvalid, Q) are zero-filled with ordinary LDS stores.  Every wave issues
// whole 1 KB blocks: block k covers LDS slots [64 k, 64 k + 64), lane l fills
// slot 64 k + l (row slot / CPR, physical chunk slot % CPR) from the global
// chunk that the swizzle puts there.
template <int Q, int W, int CPR>
__device__ inline void stage_rows_async(bf16 *lds, const bf16 *src, int64_t gstride, int nvalid,
                                        int wave, int lane, int tid) {
    constexpr int nblk = Q * CPR / 64;
    static_assert(Q * CPR % 64 == 0, "whole 1 KB blocks");
    for (int k = wave; k < nblk; k += W) {
        const int slot = k * 64 + lane;
        const int r = slot / CPR, pc = slot % CPR;
        const int c = pc ^ swz<CPR>(r);
        if (r < nvalid)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + (int64_t)r * gstride + c * 8),
                (__attribute__((address_space(3))) void *)(lds + k * 512), 16, 0, 0);
    }
    if (nvalid < Q) {
        for (int v = tid; v < (Q - nvalid) * CPR; v += 64 * W)
            *(bf16x8 *)&lds[(nvalid * CPR + v) * 8] = bf16x8{};
    }
}

template <int Q, int N, int PB>
__global__ __launch_bounds__(64 * ((Q == 256) ? 8 : 4)) void ssd_chunk_bf16_kernel(ChunkArgs a) {
    using Cfg = Bf16Cfg<Q, N, PB>;
    constexpr int W = Cfg::W, THREADS = Cfg::THREADS;
    constexpr int NT = Cfg::NT, PT = Cfg::PT, KN = Cfg::KN, IT = Cfg::IT;
    constexpr int ST = Cfg::ST, NTW = Cfg::NTW, PTW = Cfg::PTW;
    constexpr int CPRB = Cfg::CPRB, CPRX = Cfg::CPRX, LDH = Cfg::LDH, XBUF = Cfg::XBUF;
    static_assert(Cfg::kLdsBytes <= 160 * 1024, "LDS budget");
    static_assert(THREADS == 64 * ((Q == 256) ? 8 : 4), "launch bounds");

    __shared__ __attribute__((aligned(1024))) bf16 sB[Cfg::SB];
    __shared__ __attribute__((aligned(1024))) bf16 sXbuf[XBUF * Cfg::SX];
    __shared__ __attribute__((aligned(16))) bf16 sH[PB * LDH];
    __shared__ __attribute__((aligned(16))) SegLds<Q> sg;
    __shared__ int s_wave_reset[W];

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
    const int c_begin = s * a.split_chunks;
    const int c_end = min(a.nchunks, c_begin + a.split_chunks);

    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.f;
    const float *dt_row = a.dt + (int64_t)b * L * H + h;
    const int32_t *seq_row = a.seq_idx ? a.seq_idx + (int64_t)b * L : nullptr;
    const int p_base = pb * PB;
    const bf16 *Bsrc = (const bf16 *)a.B + ((int64_t)b * L * G + grp) * N;
    const bf16 *Csrc = (const bf16 *)a.C + ((int64_t)b * L * G + grp) * N;
    const bf16 *Xsrc = (const bf16 *)a.x + ((int64_t)b * L * H + h) * P + p_base;

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

    // ---- the next chunk's C rows and token values, prefetched into registers
    bf16x8 cf[IT][KN];     // C_c rows of this wave's row tiles (B operand, k = n)
    bf16x8 pC[IT][KN];
    float p_dt = 0.f;
    int p_flag = 0;
    auto prefetch_regs = [&](int c) {
        const int t0 = c * Q;
        const int nvalid = min(Q, L - t0);
        if (full) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int i = row_tile<Cfg>(wave, it) * 16 + l16;
#pragma unroll
                for (int kk = 0; kk < KN; ++kk) {
                    const int col = kk * 32 + 8 * g;
                    pC[it][kk] = load8(Csrc + (int64_t)(t0 + i) * G * N + col, i < nvalid && col < N);
                }
            }
        }
        if (tid < Q) seg_fetch_token(tid, t0, nvalid, dt_row, H, seq_row, p_dt, p_flag);
    };
    auto stage_x = [&](int c) {
        const int t0 = c * Q;
        stage_rows_async<Q, W, CPRX>(sXbuf + (XBUF == 2 ? (c & 1) : 0) * Cfg::SX,
                                     Xsrc + (int64_t)t0 * H * P, (int64_t)H * P, min(Q, L - t0),
                                     wave, lane, tid);
    };
    auto stage_b = [&](int c) {
        const int t0 = c * Q;
        stage_rows_async<Q, W, CPRB>(sB, Bsrc + (int64_t)t0 * G * N, (int64_t)G * N,
                                     min(Q, L - t0), wave, lane, tid);
    };

    if (c_begin < c_end) {
        stage_x(c_begin);
        stage_b(c_begin);
        prefetch_regs(c_begin);
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * Q;
        const int nvalid = min(Q, L - t0);
        const bf16 *sX = sXbuf + (XBUF == 2 ? (c & 1) : 0) * Cfg::SX;

        // ---- 1. token values and C rows of this chunk (prefetched one chunk ago)
        if (full) {
#pragma unroll
            for (int it = 0; it < IT; ++it)
#pragma unroll
                for (int kk = 0; kk < KN; ++kk) cf[it][kk] = pC[it][kk];
        }
        int flag = 0;
        if (tid < Q) {
            seg_store_token<Q>(sg, tid, p_dt, A_h, p_flag);
            flag = p_flag;
        }
        const unsigned long long wave_flags = __ballot(flag);
        if (lane == 0) s_wave_reset[wave] = wave_flags != 0ull;
        lds_sync();

        // ---- 3. segsum factors
        if (tid == 0) {
            int any = 0;
#pragma unroll
            for (int w2 = 0; w2 < W; ++w2) any |= s_wave_reset[w2];
            sg.any_reset = any;
        }
        if (tid < Q) seg_block_sums<Q>(sg, tid);
        lds_sync();
        if (tid < Q) seg_chunk_products<Q>(sg, tid);
        // X_c and B_c have landed (and every wave is past the segsum steps)
        vmem_lds_sync();

        // ---- 2. next chunk's X tile and register values go out now
        if (c + 1 < c_end) {
            if (XBUF == 2) stage_x(c + 1);
            prefetch_regs(c + 1);
        }

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
            // Y^T = h^T C^T  (A = h^T rows p, B = C rows i; k = n)
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
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
            for (int it = 0; it < IT; ++it) {
                const int I = row_tile<Cfg>(wave, it);
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
                const int rr = jr0 + (l16 >> 2), col = pt * 16 + 4 * (l16 & 3);
                xa[pt] = join_bf16x8(lds_read_tr16(&sX[tile_off_col<CPRX>(rr, col)]),
                                     lds_read_tr16(&sX[tile_off_col<CPRX>(rr + 16, col)]));
            }
            // chunk state: h += (B_c^T diag(w dt)) X_c over these 32 tokens
            if (st_valid) {
                const f32x4 w0 = *(const f32x4 *)&sg.wcd[jr0];
                const f32x4 w1 = *(const f32x4 *)&sg.wcd[jr0 + 16];
#pragma unroll
                for (int an = 0; an < NTW; ++an) {
                    const int nt = nt0 + an;
                    const int rr = jr0 + (l16 >> 2), col = nt * 16 + 4 * (l16 & 3);
                    const bf16x8 raw = join_bf16x8(lds_read_tr16(&sB[tile_off_col<CPRB>(rr, col)]),
                                                   lds_read_tr16(&sB[tile_off_col<CPRB>(rr + 16, col)]));
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
            if (row_tile<Cfg>(wave, IT - 1) < 2 * m && row_tile<Cfg>(wave, 0) < 2 * m) continue;
            const f32x4 dt0 = *(const f32x4 *)&sg.dt[jr0];
            const f32x4 dt1 = *(const f32x4 *)&sg.dt[jr0 + 16];
            const f32x4 W0 = *(const f32x4 *)&sg.W[jr0];
            const f32x4 W1 = *(const f32x4 *)&sg.W[jr0 + 16];
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int I = row_tile<Cfg>(wave, it);
                if (I < 2 * m) continue;
                const int i = I * 16 + l16;
                // mask times dt for both 16-token halves (zero above the diagonal);
                // the F chain runs leftwards, so the upper half goes first
                float sc[2][4];
#pragma unroll
                for (int hf = 1; hf >= 0; --hf) {
                    const int jt = 2 * m + hf;
                    const f32x4 dtv = hf ? dt1 : dt0;
                    const f32x4 Wv = hf ? W1 : W0;
                    float Lr[4] = {0.f, 0.f, 0.f, 0.f};
                    if (jt == I) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            Lr[r] = seg_diag_value(ediag[it][r], i, jt * 16 + 4 * g + r, rs_i[it]);
                    } else if (jt < I) {
                        if (jt < I - 1) Fch[it] = seg_chain_step(Fch[it], sg.Tb[jt + 1]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) Lr[r] = seg_offdiag(Fch[it], Wv[r]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) sc[hf][r] = Lr[r] * dtv[r];
                }
                // S^T tiles of both halves
                f32x4 S[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int jt = 2 * m + hf;
                    S[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (jt > I) continue;
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) {
                        const int ch = kk * 4 + g;
                        const bf16x8 bfrag = load8(&sB[tile_off<CPRB>(jt * 16 + l16, ch & (CPRB - 1))],
                                                   ch < CPRB);
                        S[hf] = kk == 0 ? mfma_bf16_zero_acc(bfrag, cf[it][0])
                                        : mfma_bf16(bfrag, cf[it][kk], S[hf]);
                    }
                }
                mfma_fence(S[0], S[1]);
                bf16x8 pf;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int r = 0; r < 4; ++r) pf[hf * 4 + r] = (bf16)(S[hf][r] * sc[hf][r]);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[it][pt] = mfma_bf16(xa[pt], pf, acc[it][pt]);
            }
        }

        mfma_fence_all(hs);
        if (full) {
#pragma unroll
            for (int it = 0; it < IT; ++it) mfma_fence_all(acc[it]);
            bf16 *yg = (bf16 *)a.y;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int i = row_tile<Cfg>(wave, it) * 16 + l16;
                if (i >= nvalid) continue;
                bf16 *yrow = yg + (((int64_t)b * L + t0 + i) * H + h) * P + p_base;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int p = pt * 16 + 4 * g;
                    const bf16x4 xv = *(const bf16x4 *)&sX[tile_off_col<CPRX>(i, p)];
                    f32x4 o = acc[it][pt];
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] += D_h * (float)xv[r];
                    *(bf16x4 *)(yrow + p) = f32x4_to_bf16x4(o);
                }
            }
        }
        lds_sync();   // all reads of sB, sX, sH and the segsum values are done
        if (c + 1 < c_end) {
            if (XBUF == 1) stage_x(c + 1);
            stage_b(c + 1);
        }
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
