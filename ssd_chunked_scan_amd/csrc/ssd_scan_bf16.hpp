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
// loaded here.  Neither is scaled here: the decays go onto X and onto the
// accumulators.
//
// Decay factorisation (page "GPU Hierarchy Meets Structured Matrices": the
// mask is 1-semiseparable, so an off-diagonal sub-block is rank one).  With
// 16-token sub-blocks, Tb_K the decay over sub-block K, W_j the decay from
// token j to the end of its sub-block and F_i the decay from the start of row
// i's sub-block I through i, an entry of sub-block (I, J), J < I, is
//
//   L_ij dt_j = F_i * (Tb_{J+1} ... Tb_{I-1}) * W_j dt_j.
//
// The middle product does not depend on i or j.  Over 32-token column pairs
// m (sub-blocks 2m, 2m+1; one MFMA K step) it is built by Horner's rule: with
// X''_j = W_j dt_j x_j, times Tb_{J+1} when J is even (the first sub-block of
// its pair),
//
//   acc <- acc * (Tb_{2m} Tb_{2m+1}) + (C B^T)_{I, pair m} X''_{pair m}
//
// run over the pairs left of row tile I's diagonal pair, starting from the
// state projection, leaves every term with its middle product (and the
// projection with Tb_0 ... Tb_{I-1}); one more factor Tb_{I-1} for odd I and
// the row factor F_i finish it.  The chunk state takes the same recurrence
// over all pairs, starting from h_{c-1}: the pair decays then multiply out to
// the decay from each token to the chunk end.  Every factor is a product of
// decays in [0, 1] (no division, no exp of a positive sum), so the recurrence
// is as stable as the direct product.  Only the diagonal pair of each row
// tile is masked element by element (with the unscaled X); D x rides on its
// diagonal.
//
// Everything is computed transposed (rows = headdim p) so that each lane of
// an output tile owns one token i and four consecutive p: the row factor F_i
// is one value per lane and y is written 8 bytes per lane.
//
// MFMA 16x16x32 bf16 operand layout (verified on gfx950): A (16 x 32):
// lane l holds row l%16, k = 8(l/16)..+7; B (32 x 16): lane l holds column
// l%16, the same k; D (16 x 16): lane l holds column l%16, rows 4(l/16)..+3.
// Over tokens (k = j) both operands use the slot map
// e -> j = j0 + 4g + (e%4) + 16(e/4), g = l/16.
//
// Work split inside the workgroup: W waves (8 for Q = 256, else 4).  Output
// rows (16-token tiles) are dealt in the pairs (w, Q/16-1-w) so every wave
// gets the same number of lower-triangular tiles; state tiles (16 x 16 of
// N x P) are split by n first.
//
// Wave roles.  Vector-memory loads and stores of one wave complete in issue
// order, so a wave that has a slow HBM load or a scattered store in flight
// cannot use any load it issued later.  All HBM traffic of the workgroup is
// therefore issued by extra producer waves (4 at Q = 256, else 2), and the
// W compute waves only load operands that the other heads of the row keep in
// L2 (C B^T, B^T and C rows).  During chunk c the producers store y_{c-1}
// (rows of 16-byte chunks read from an LDS tile; times silu(z_{c-1}) when the
// output gate is fused), issue the direct-to-LDS loads
// (global_load_lds_dwordx4) of X_{c+1}, gather dt of chunk c+1 (through the
// fused dt map) and compute its segsum values (page "GPU Hierarchy Meets
// Structured Matrices": the sub-block sums) into the other half of a double
// buffer.  Four producers rather than two at Q = 256: the same time without
// the gate (145 us at the 2.7B layer either way), 249 -> 217 us with it.
//
// Per chunk, two barriers.  Between them X_{c+1} is turned into MFMA
// fragments once for all compute waves (unscaled and X'', fragment-ordered so
// that each operand is one 16-byte LDS read per lane), and h_c and y_c go to
// LDS as bf16 (the producers store y_c during chunk c+1).  The first pair's
// fragments and the C rows of chunk c+1 go out last before the first barrier
// and stay in flight across it (its wait counts them out); the C B^T and B^T
// fragments of the other pairs are loaded two pairs ahead of their use
// (one pair ahead: 193.6 -> 190.7 us cold forward at the 2.7B layer, the
// 32-head chunk-128 sweep 152.6 -> 145.2 us; three ahead spill).
#pragma once

#include <type_traits>

#include "ssd_common.hpp"
#include "ssd_segsum.hpp"
#include "ssd_tiles.hpp"

namespace ssd {

#ifndef SSD_PRODUCER_INFLIGHT
#define SSD_PRODUCER_INFLIGHT 32
#endif
#ifndef SSD_PAIR_PREFETCH
#define SSD_PAIR_PREFETCH 2
#endif
#ifndef SSD_NPROD_Q256
#define SSD_NPROD_Q256 4
#endif

template <int Q, int N, int PB>
struct ScanCfg {
    static constexpr int W = (Q == 256) ? 8 : 4;        // compute waves
    static constexpr int NPROD = (Q == 256) ? SSD_NPROD_Q256 : 2;   // producer waves
    static constexpr int THREADS = 64 * (W + NPROD);
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
    static constexpr int NFRAG = NP * PT;                // X fragments (pair, headdim tile)
    static constexpr int LDH = N + 8;                    // padded pitch of the h^T tile
    static constexpr int NYB = Q * PB * 2 / 1024;        // 1 KB blocks of the y tile
    static constexpr int NBLK = CbShape<Q>::NBLK;
    // X stage, two fragment sets, y tile, h tile, segsum values
    static constexpr size_t kLdsBytes =
        4 * (size_t)SX * 2 + (size_t)PB * LDH * 2 + 2 * sizeof(SegBuf<Q>);
    static_assert(Q % 64 == 0 && Q <= 256, "chunk size");
    static_assert(NPROD == 2 || NPROD == 4, "producer waves");
    static_assert(N % 16 == 0 && N <= 128, "dstate");
    static_assert(PB % 16 == 0 && PB <= 128, "headdim block");
    static_assert(ST % NTW == 0, "state tile split");
    static_assert(IT == 1 || TILES == 2 * W, "row tile pairs");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// One workgroup's walk over its chunks.  PB is the number of headdim columns
// the workgroup owns (a whole headdim block, or half of one); the LDS arrays
// belong to the kernel and are at least as large as this PB needs.
//
// SEG selects how the output path evaluates the intra-chunk mask (segsum
// ablation, page "GPU Hierarchy Meets Structured Matrices", abstract):
// kSegsumHierarchy is the factorisation above.  kSegsumDirect and
// kSegsumDiff mask every 32-token block of C B^T left of and on the diagonal
// element by element, L_ij dt_j with L_ij = 2^s_ij, and multiply the unscaled
// X: direct takes s_ij as its own running sum d_i + d_{i-1} + ... + d_{j+1}
// (each lane walks its row leftwards from the diagonal), diff as cs_i - cs_j
// of the chunk's inclusive prefix sums cs (an associative scan, in vcs).  The
// state path, the row factor of the state projection and the chunk decay are
// the hierarchy's in all three, so that only the mask evaluation differs.
template <int Q, int N, int PB, bool LOCAL, int SEG>
__device__ __attribute__((always_inline)) inline void scan_body(
        const ChunkArgs &a, const Unit un, const int p_base, bf16 *__restrict__ sXstage,
        bf16x8 *__restrict__ sXr, bf16x8 *__restrict__ sXs, bf16 *__restrict__ sY,
        bf16 *__restrict__ sH, SegBuf<Q> *__restrict__ segbuf, bf16x8 *__restrict__ sTouch,
        float *__restrict__ vcs) {
    using Cfg = ScanCfg<Q, N, PB>;
    constexpr int W = Cfg::W, THREADS = Cfg::THREADS;
    constexpr int NT = Cfg::NT, PT = Cfg::PT, KN = Cfg::KN, IT = Cfg::IT, NP = Cfg::NP;
    constexpr int ST = Cfg::ST, NTW = Cfg::NTW, PTW = Cfg::PTW, NFRAG = Cfg::NFRAG;
    constexpr int CPRX = Cfg::CPRX, LDH = Cfg::LDH, NBLK = Cfg::NBLK, NYB = Cfg::NYB;
    constexpr int CPRY = PB / 8;
    constexpr int NPROD = Cfg::NPROD;
    static_assert(THREADS == 64 * (((Q == 256) ? 8 + SSD_NPROD_Q256 : 4 + 2)), "launch bounds");
    constexpr bool kVar = SEG != kSegsumHierarchy;   // per-element mask on the output path
    static_assert(!kVar || (Q == 256 && !LOCAL && NP == W), "mask variants: chunk 256, full pass");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave >= W;
    const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int b = un.b, h = un.h, s = un.s, pb = un.pb;
    // The last split's local summary is never used (its entering state comes
    // from the scan and its end state is the final state).
    if (a.mode == kModeSplitLocal && s == a.nsplits - 1) return;
    const int L = a.seqlen, H = a.nheads, G = a.ngroups, P = a.headdim;
    const int grp = h / (H / G);
    constexpr bool full = !LOCAL;   // LOCAL: split-local pass (end state and decay only)
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
    const int64_t bg = (int64_t)b * G + grp;
    const bf16x8 *Sws = (const bf16x8 *)a.ws_S + bg * a.nchunks * NBLK * 64 + lane;
    const bf16x8 *BTws = (const bf16x8 *)a.ws_BT + bg * a.nchunks * NP * N * 4;
    const bf16x8 *Cws = (const bf16x8 *)a.ws_C + bg * a.nchunks * Cfg::TILES * KN * 64 + lane;


    // ================= producer waves =================
    // Producer pw (wave W + pw) streams blocks [pw, pw+1) * NYB / NPROD of
    // each tile and the segsum rounds k = pw mod NPROD (64 tokens each).
    auto run_producer = [&](auto PW) __attribute__((always_inline)) {
        constexpr int pw = decltype(PW)::value;
        constexpr int KB0 = pw * NYB / NPROD, KB1 = (pw + 1) * NYB / NPROD;
        const bf16 *Xsrc = (const bf16 *)a.x + ((int64_t)b * L * H + h) * P + p_base;
        // raw dt -> step size (fused prologue: bias, softplus, clamp)
        const DtMap dm = dt_map_of(a, h);
        // token values of a chunk, lane k*64+l holds token k*64+l
        float p_dt[Q / 64];
        int p_cur[Q / 64], p_prev[Q / 64];
        auto fetch_tokens = [&](int c) __attribute__((always_inline)) {
#pragma unroll
            for (int k = pw; k < Q / 64; k += NPROD) {
                const int tg = min(c * Q + k * 64 + lane, L - 1);
                p_dt[k] = dt_row[(int64_t)tg * H];
                p_cur[k] = seq_row[tg];
                p_prev[k] = seq_row[max(tg - 1, 0)];
            }
        };
        // Debug export of the factors (full pass, one workgroup per head).
        const bool dbg = !LOCAL && a.dbg_seg != nullptr && pb == 0 && un.half <= 0;
        auto segsum = [&](int c, SegBuf<Q> &sgb) __attribute__((always_inline)) {
            float *rec = dbg ? a.dbg_seg + (((int64_t)b * H + h) * a.nchunks + c) * SegRecord<Q>::WORDS
                             : nullptr;
#pragma unroll
            for (int k = pw; k < Q / 64; k += NPROD) {
                const int t = k * 64 + lane, tg = c * Q + t;
                const bool valid = tg < L;
                const float dtv = valid ? dt_apply(dm, p_dt[k]) : 0.f;
                const int flag = (resets && valid && tg > 0 && p_cur[k] != p_prev[k]) ? 1 : 0;
                seg_tokens<Q>(sgb, t, dtv, flag, A_h, resets, rec);
            }
        };
        // HBM streams of the workgroup in 1 KB blocks (64 lanes x 16 bytes):
        // block k of X_c goes straight to LDS (sXstage, swizzled, rows past
        // the sequence end read zeros), block k of the y tile of chunk c goes
        // from sY to global memory.  Lane l of block k is physical chunk
        // 64k + l of the tile: row r = (64k + l) / CPR, logical chunk
        // ((64k + l) % CPR) ^ swz(r).
        // Per lane: row lane / CPR of each block and its byte offset, fixed
        // for the whole kernel; per block: a uniform row base and the
        // swizzled chunk (k is a compile-time constant after unrolling).
        const uint32_t row_bytes = (uint32_t)H * P * 2;
        const int xrow = lane / CPRX, xpc = lane % CPRX;
        const int yrow = lane / CPRY, ypc = lane % CPRY;
        const uint32_t xrow_off = (uint32_t)xrow * row_bytes, yrow_off = (uint32_t)yrow * row_bytes;
        const char *xbase = (const char *)Xsrc;
        char *ybase = (char *)a.y + ((((int64_t)b * L) * H + h) * P + p_base) * 2;
        auto dma_to = [&](const char *src, bf16 *dst) __attribute__((always_inline)) {
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
        };
        auto dma_x = [&](int c, int k) __attribute__((always_inline)) {
            constexpr int RB = 64 / CPRX;   // rows per block
            const int t0 = c * Q, r = k * RB + xrow;
            const int cc = xpc ^ swz<CPRX>(r);
            const char *src = xbase + (int64_t)(t0 + k * RB) * row_bytes + (xrow_off + cc * 16);
            if (t0 + Q > L && t0 + r >= L) src = (const char *)kZeroChunk;
            dma_to(src, sXstage + k * 512);
        };
        // Split-local pass: X_c goes to staging buffer c mod 3 (sXstage, or
        // the unscaled fragment set and the y tile, which that pass does not
        // use).  The buffer is a compile-time choice, so that every
        // asynchronous load names its LDS object and offset (the compiler
        // then sees that the loads of one tile do not overlap).
        auto stream_local = [&](int cx, auto BUF) __attribute__((always_inline)) {
            constexpr int bsel = decltype(BUF)::value;
            bf16 *base = bsel == 0 ? sXstage : (bsel == 1 ? (bf16 *)sXr : sY);
            constexpr int RB = 64 / CPRX;
            const int t0 = cx * Q;
#pragma unroll
            for (int k = KB0; k < KB1; ++k) {
                const int r = k * RB + xrow;
                const int cc = xpc ^ swz<CPRX>(r);
                const char *src = xbase + (int64_t)(t0 + k * RB) * row_bytes + (xrow_off + cc * 16);
                if (t0 + Q > L && t0 + r >= L) src = (const char *)kZeroChunk;
                dma_to(src, base + k * 512);
            }
        };
        // X_cx into its buffer; with WAIT, then the barrier that leaves
        // exactly those loads in flight (the marker differs per buffer so
        // that the three copies stay separate straight-line code).
        auto prefetch_local = [&](int cx, bool wait) __attribute__((always_inline)) {
            constexpr int KB = KB1 - KB0;
            const int sel = cx % 3;
            if (sel == 0) {
                stream_local(cx, std::integral_constant<int, 0>{});
                if (wait) vmem_lds_sync_lookahead<KB, 0>();
            } else if (sel == 1) {
                stream_local(cx, std::integral_constant<int, 1>{});
                if (wait) vmem_lds_sync_lookahead<KB, 1>();
            } else {
                stream_local(cx, std::integral_constant<int, 2>{});
                if (wait) vmem_lds_sync_lookahead<KB, 2>();
            }
        };
        // Fused output gate: z of chunk c is loaded (16 bytes per lane and
        // block, unconditionally: rows past the sequence end read zeros)
        // while chunk c is computed, and multiplies y_c, as silu(z), when
        // y_c is stored during chunk c+1.  The gate acts on the bf16 y tile.
        const bool gated = a.z != nullptr;
        const char *zbase = gated ? (const char *)a.z + ((((int64_t)b * L) * H + h) * P + p_base) * 2
                                  : (const char *)kZeroChunk;
        bf16x8 zr[KB1 - KB0];
        auto load_z = [&](int c, int k) __attribute__((always_inline)) {
            constexpr int RB = 64 / CPRY;
            const int t0 = c * Q, r = k * RB + yrow;
            const int cc = ypc ^ swz<CPRY>(r);
            const char *src = zbase + (int64_t)(t0 + k * RB) * row_bytes + (yrow_off + cc * 16);
            if (t0 + Q > L && t0 + r >= L) src = (const char *)kZeroChunk;
            // a global load: z and the zero chunk are both global memory, but
            // the select of the two would otherwise be a flat load, which also
            // counts against the LDS wait counter
            zr[k - KB0] = *(const __attribute__((address_space(1))) bf16x8 *)src;
        };
        auto store_y = [&](int c, int k) __attribute__((always_inline)) {
            constexpr int RB = 64 / CPRY;
            const int t0 = c * Q, r = k * RB + yrow;
            const int cc = ypc ^ swz<CPRY>(r);
            bf16x8 v = *(const bf16x8 *)&sY[(k * 64 + lane) * 8];
            if (gated) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float zf = (float)zr[k - KB0][e];
                    v[e] = (bf16)((float)v[e] * silu_f32(zf));
                }
            }
            char *dst = ybase + (int64_t)(t0 + k * RB) * row_bytes + (yrow_off + cc * 16);
            // non-temporal: y is not read again here, and plain stores of it
            // cost the L2-resident per-group operands (measured 207 -> 171 us
            // at layer27b; the same hint on the X loads loses it again)
            if (t0 + Q <= L || t0 + r < L) __builtin_nontemporal_store(v, (bf16x8 *)dst);
        };
        // Both streams, interleaved, with at most kInFlight blocks
        // outstanding: a steady trickle keeps HBM busy without filling the
        // memory pipeline that the compute waves' L2 loads go through.
        constexpr int kGroup = (KB1 - KB0) < 4 ? (KB1 - KB0) : 4, kInFlight = SSD_PRODUCER_INFLIGHT;
        static_assert((KB1 - KB0) % kGroup == 0 && NYB % NPROD == 0, "whole groups");
        // cz >= 0: also load z of chunk cz (after block k of y_cy has taken
        // the z of chunk cy from the same registers).
        auto stream = [&](int cx, int cy, int cz) __attribute__((always_inline)) {
#pragma unroll
            for (int k0 = KB0; k0 < KB1; k0 += kGroup) {
#pragma unroll
                for (int k = k0; k < k0 + kGroup; ++k) {
                    if (cx >= 0) dma_x(cx, k);
                    if (cy >= 0) store_y(cy, k);
                    if (cz >= 0) load_z(cz, k);
                }
                if (k0 + kGroup < KB1) {
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    __builtin_amdgcn_s_waitcnt(wait_vm(kInFlight));
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                }
            }
        };

        // chunk c: X_{c+1} and y_{c-1} (written to sY by the compute waves
        // between the barriers of the previous hand-over), the segsum of
        // chunk c+1 from token values gathered during chunk c-1, and the
        // gather of chunk c+2's token values after the first barrier.
        if constexpr (LOCAL) {
            // Split-local pass: X runs two chunks ahead (three staging
            // buffers), because this pass has too little work per chunk to
            // cover an HBM round trip.  At the first barrier of chunk c only
            // X_{c+1} must have landed: the loads of X_{c+2}, issued last,
            // may still be in flight (completions count in issue order).
            // The token values of chunk c+1 are gathered one chunk ahead of
            // its segsum: issued after the barrier that waits for X_{c+1} in
            // the walk of chunk c-1, so that the segsum does not wait for
            // their round trip (this pass has little else to hide it behind).
            fetch_tokens(c_begin);
            prefetch_local(c_begin, false);
            segsum(c_begin, segbuf[c_begin & 1]);
            if (c_begin + 1 < c_end) prefetch_local(c_begin + 1, true);   // X_{c_begin} has landed
            else vmem_lds_sync();
            if (c_begin + 1 < c_end) fetch_tokens(c_begin + 1);
            lds_sync();
            for (int c = c_begin; c < c_end; ++c) {
                if (c + 1 < c_end) segsum(c + 1, segbuf[(c + 1) & 1]);
                if (c + 2 < c_end) prefetch_local(c + 2, true);   // X_{c+1} has landed
                else vmem_lds_sync();
                if (c + 2 < c_end) fetch_tokens(c + 2);
                lds_sync();
            }
            return;
        }
        fetch_tokens(c_begin);
        stream(c_begin, -1, -1);
        segsum(c_begin, segbuf[c_begin & 1]);
        vmem_lds_sync();
        if (c_begin + 1 < c_end) fetch_tokens(c_begin + 1);
        lds_sync();
        // y_{c-1} of a whole chunk in straight-line, unpredicated stores (the
        // blocks are issued in the same order as by stream)
        auto store_y_whole = [&](int cy) __attribute__((always_inline)) {
#pragma unroll
            for (int k = KB0; k < KB1; ++k) {
                constexpr int RB = 64 / CPRY;
                const int t0 = cy * Q, r = k * RB + yrow;
                const int cc = ypc ^ swz<CPRY>(r);
                const bf16x8 v = *(const bf16x8 *)&sY[(k * 64 + lane) * 8];
                char *dst = ybase + (int64_t)(t0 + k * RB) * row_bytes + (yrow_off + cc * 16);
                __builtin_nontemporal_store(v, (bf16x8 *)dst);
            }
        };
        // With the output gate: block by block, y_{cy} times silu(z_{cy}) (z
        // from the registers that the loads of the previous chunk filled),
        // then the loads of z_cz into the same registers.
        auto store_y_whole_gated = [&](int cy, int cz) __attribute__((always_inline)) {
#pragma unroll
            for (int k = KB0; k < KB1; ++k) {
                constexpr int RB = 64 / CPRY;
                const int t0 = cy * Q, r = k * RB + yrow;
                const int cc = ypc ^ swz<CPRY>(r);
                bf16x8 v = *(const bf16x8 *)&sY[(k * 64 + lane) * 8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (bf16)((float)v[e] * silu_f32((float)zr[k - KB0][e]));
                char *dst = ybase + (int64_t)(t0 + k * RB) * row_bytes + (yrow_off + cc * 16);
                __builtin_nontemporal_store(v, (bf16x8 *)dst);
                load_z(cz, k);
            }
        };
        // L2 prefetches of this producer's blocks of X_{c+2} (direct-to-LDS
        // loads into sTouch, which nothing reads), issued after the loads of
        // X_{c+1} and left in flight across the hand-over: the loads of
        // X_{c+2} during chunk c+1 then find them in L2 (measured at the 2.7B
        // layer, cold: forward 209 -> 201 us).  The per-group operands are not
        // prefetched: in the forward pass the per-group kernel has just written
        // them to L2, and a slice-wise prefetch of them only added traffic
        // (201 -> 197 us).
        auto touch_x = [&](int cx) __attribute__((always_inline)) {
            constexpr int RB = 64 / CPRX;
#pragma unroll
            for (int k = KB0; k < KB1; ++k) {
                const int t0 = cx * Q, r = k * RB + xrow;
                const int cc = xpc ^ swz<CPRX>(r);
                const char *src = xbase + (int64_t)(t0 + k * RB) * row_bytes + (xrow_off + cc * 16);
                if (t0 + Q > L && t0 + r >= L) src = (const char *)kZeroChunk;
                l2_touch(src, sTouch);
            }
        };
        for (int c = c_begin; c < c_end; ++c) {
            const bool more = c + 1 < c_end;
            if (gated) {
                // With the output gate, in steady state as below: X_{c+1}, the
                // segsum of chunk c+1, then, in flight across the barrier, the
                // prefetches of X_{c+2}, the gated stores of y_{c-1} and the
                // loads of z_c (used when y_c is stored during chunk c+1).
                // Measured at the 2.7B layer, cold: 245 -> 226 us (every one of
                // them had been waited for at the barrier; without the z loads
                // 198 us).  An L2 prefetch of z_{c+1} as well: +9 us.
                const int cy = c - 1;
                if (more && c > c_begin && (cy + 1) * Q <= L) {
                    stream(c + 1, -1, -1);
                    segsum(c + 1, segbuf[(c + 1) & 1]);
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    touch_x(min(c + 2, c_end - 1));
                    store_y_whole_gated(cy, c);
                    vmem_lds_sync_touch<3 * (KB1 - KB0)>();
                } else {
                    stream(more ? c + 1 : -1, c > c_begin ? c - 1 : -1, c);
                    if (more) segsum(c + 1, segbuf[(c + 1) & 1]);
                    vmem_lds_sync();   // X_{c+1} and z_c have landed, sY is read
                }
                if (c + 2 < c_end) fetch_tokens(c + 2);
                lds_sync();        // the compute waves write y_c to sY in between
                continue;
            }
            // Without the gate: X_{c+1} first, then the segsum of chunk c+1
            // (its token values were gathered after the previous chunk's
            // first barrier, one chunk ahead, as in the split-local pass:
            // packed 334 -> 319 us, decay stress 174 -> 167 us of the
            // forward pass), then the stores of y_{c-1}.  The barrier needs
            // X_{c+1} in LDS and the y tile read out of sY, not the stores'
            // completions: for a whole chunk it lets exactly those KB1 - KB0
            // newest operations, the stores, stay in flight (completions
            // count in issue order).
            if (more) {
                stream(c + 1, -1, -1);
                segsum(c + 1, segbuf[(c + 1) & 1]);
            }
            const int cy = c - 1;
            if (more && c > c_begin && (cy + 1) * Q <= L) {
                // in flight across the barrier: the prefetches of X_{c+2}
                // and the stores of y_{c-1}
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                touch_x(min(c + 2, c_end - 1));
                store_y_whole(cy);
                vmem_lds_sync_touch<2 * (KB1 - KB0)>();
            } else {
                if (c > c_begin) stream(-1, cy, -1);
                vmem_lds_sync();
            }
            if (c + 2 < c_end) fetch_tokens(c + 2);
            lds_sync();        // the compute waves write y_c to sY in between
        }
        stream(-1, c_end - 1, -1);
        // nothing may land in this workgroup's LDS after it ends
        __builtin_amdgcn_s_waitcnt(kWaitVmemLgkm0);
    };
    if (producer) {
        if (wave == W) run_producer(std::integral_constant<int, 0>{});
        else if (NPROD == 2 || wave == W + 1) run_producer(std::integral_constant<int, 1>{});
        else if (wave == W + 2) run_producer(std::integral_constant<int, (NPROD > 2) ? 2 : 0>{});
        else run_producer(std::integral_constant<int, (NPROD > 3) ? 3 : 0>{});
        return;
    }

    // ================= compute waves =================
    // The compute waves hold the critical path of every chunk: they issue
    // ahead of the producer waves on their SIMD (measured at the 2.7B layer,
    // cold: 198 -> 196 us; the producers ahead instead: 202 us).
    __builtin_amdgcn_s_setprio(1);
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

    auto write_h = [&]() __attribute__((always_inline)) {
        if (!full || !st_valid) return;
#pragma unroll
        for (int k = 0; k < ST; ++k) {
            const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
            *(bf16x4 *)&sH[(pt * 16 + l16) * LDH + nt * 16 + 4 * g] = f32x4_to_bf16x4(hs[k]);
        }
    };
    // sXstage -> fragments (between the two barriers of a hand-over): fragment
    // (m, pt) holds, for lane (p = 16 pt + l16, g), X[j][p] at the slot tokens
    // j = 32m + 4g + (e%4) + 16(e/4); sXs holds the same times the X'' factor.
    auto make_fragments_from = [&](const SegBuf<Q> &sg, const bf16 *xs_src) __attribute__((always_inline)) {
        // wave w makes the fragments of pairs w, w + W, ...: the pair's X''
        // factors are read and multiplied once for all its headdim tiles
#pragma unroll
        for (int m0 = 0; m0 < NP; m0 += W) {
            const int m = m0 + wave;
            if (NP % W != 0 && m >= NP) break;
            const int jr = 32 * m + 4 * g;
            const f32x4 wlo = *(const f32x4 *)&sg.wd[jr];
            const f32x4 whi = *(const f32x4 *)&sg.wd[jr + 16];
            const float tb_hi = sg.Tb[2 * m + 1];
            float flo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) flo[r] = __fmul_rn(wlo[r], tb_hi);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int rr = jr + (l16 >> 2), col = pt * 16 + 4 * (l16 & 3);
                const bf16x8 xr = join_bf16x8(lds_read_tr16(&xs_src[tile_off_col<CPRX>(rr, col)]),
                                              lds_read_tr16(&xs_src[tile_off_col<CPRX>(rr + 16, col)]));
                bf16x8 xs;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xs[r] = (bf16)((float)xr[r] * flo[r]);
                    xs[4 + r] = (bf16)((float)xr[4 + r] * whi[r]);
                }
                if constexpr (!LOCAL) sXr[(m * PT + pt) * 64 + lane] = xr;   // a staging buffer when LOCAL
                sXs[(m * PT + pt) * 64 + lane] = xs;
            }
        }
    };
    auto make_fragments = [&](const SegBuf<Q> &sg, int cx) __attribute__((always_inline)) {
        // X_cx's staging buffer (always sXstage in the full pass).  One copy
        // of the code per buffer, each naming its array: a pointer selected
        // at run time was lowered to a table of generic pointers in scratch
        // memory and flat loads.
        if constexpr (LOCAL) {
            const int sel = cx % 3;
            if (sel == 0) make_fragments_from(sg, sXstage);
            else if (sel == 1) make_fragments_from(sg, (const bf16 *)sXr);
            else make_fragments_from(sg, (const bf16 *)sY);
        } else {
            make_fragments_from(sg, sXstage);
        }
    };
    // C_c rows of this wave's row tiles (B operand of the state projection,
    // k = n), in operand order from the per-group kernel (one contiguous
    // 1 KB load each; rows past the sequence end and columns past dstate are
    // zero there).
    bf16x8 cf[IT][KN];
    auto load_c = [&](int c, const int (&Irow)[IT]) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
#pragma unroll
            for (int kk = 0; kk < KN; ++kk)
                cf[it][kk] = Cws[(((int64_t)c * Cfg::TILES + Irow[it]) * KN + kk) * 64];
        }
    };
    // Output tile accumulators: acc[it][pt] = Y^T tile (rows p, columns i).
    f32x4 acc[IT][PT];
    // y tile of this wave's row tiles into sY (bf16)
    auto write_y = [&](const int (&Irow)[IT]) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < IT; ++it) mfma_fence_all(acc[it]);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = Irow[it] * 16 + l16;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                *(bf16x4 *)&sY[tile_off_col<CPRY>(i, pt * 16 + 4 * g)] = f32x4_to_bf16x4(acc[it][pt]);
        }
    };

    // Fragments of pair m of chunk c (C B^T blocks of the wave's row tiles and
    // B^T of its state n-tiles) into slot m % NS, loaded unconditionally: a row
    // tile whose diagonal pair lies left of m loads its diagonal pair again,
    // so the last load of each row tile is its diagonal pair (taking the
    // fragment from the previous slot instead, behind a branch, measured
    // slower: 197 -> 202 us at the 2.7B layer, the copy waits for the load).
    constexpr int PD = SSD_PAIR_PREFETCH;   // pairs loaded ahead of their use
    constexpr int NS = PD + 1;               // fragment slots
    bf16x8 sfr[NS][IT], bfr[NS][NTW];
    auto load_pair_of = [&](int c, int m, const int (&Irow)[IT]) __attribute__((always_inline)) {
        const bf16x8 *Sc = Sws + (int64_t)c * NBLK * 64;
        const bf16x8 *BTc = BTws + (int64_t)c * NP * N * 4;
        const int slot = m % NS;
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
    // B^T fragments of pair m alone (the mask variants load their C B^T
    // blocks in the output loop)
    auto load_bt_of = [&](int c, int m) __attribute__((always_inline)) {
        const bf16x8 *BTc = BTws + (int64_t)c * NP * N * 4;
        const int slot = m % NS;
#pragma unroll
        for (int q = 0; q < NTW; ++q)
            bfr[slot][q] = BTc[((int64_t)m * N + min(nt0 + q, NT - 1) * 16 + l16) * 4 + g];
    };
    // the first pair's fragments of chunk c, loaded before the hand-over into
    // it, and the vector-memory operations that issues
    auto load_pair0 = [&](int c, const int (&Irow)[IT]) __attribute__((always_inline)) {
        if constexpr (kVar) load_bt_of(c, 0);
        else load_pair_of(c, 0, Irow);
    };
    constexpr int kPair0Loads = (kVar ? 0 : IT) + NTW;

    // Diff segsum: the inclusive prefix sums cs of the chunk's log2-decays
    // (Kogge-Stone over the wave's lanes, four tokens per lane), computed by
    // every compute wave; wave w stores those of pair w.  Written between the
    // barriers of a hand-over, read during the next chunk.
    auto make_cs = [&](const SegBuf<Q> &sg) __attribute__((always_inline)) {
        if constexpr (SEG == kSegsumDiff) {
            const f32x4 dv = *(const f32x4 *)&sg.d[4 * lane];
            f32x4 cv;
            cv[0] = dv[0];
            cv[1] = __fadd_rn(cv[0], dv[1]);
            cv[2] = __fadd_rn(cv[1], dv[2]);
            cv[3] = __fadd_rn(cv[2], dv[3]);
            float x = cv[3];
#pragma unroll
            for (int off = 1; off < 64; off *= 2) {
                const float t = __shfl_up(x, off, 64);
                if (lane >= off) x = __fadd_rn(x, t);
            }
            float ex = __shfl_up(x, 1, 64);
            if (lane == 0) ex = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) cv[r] = __fadd_rn(ex, cv[r]);
            if ((lane >> 3) == wave) *(f32x4 *)&vcs[4 * lane] = cv;
        }
    };

    // ---- prologue: X fragments, state tile, C rows and the first pair's
    // fragments of the first chunk (the producer loads X and computes the
    // segsum values meanwhile)
    if constexpr (LOCAL) {
        vmem_lds_sync();                 // no C rows: the split-local pass has no outputs
    } else {
        load_pair0(c_begin, Irow0);
        load_c(c_begin, Irow0);
        vmem_lds_sync_keep<IT * KN + kPair0Loads>();   // C rows and pair 0 may still be in flight
    }
    if (!state_zero) write_h();
    make_cs(segbuf[c_begin & 1]);
    make_fragments(segbuf[c_begin & 1], c_begin);
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
        const SegBuf<Q> &sg = segbuf[buf];
        const int cn = min(c + 1, c_end - 1);   // next chunk (the last one repeats itself)

        // ---- 1. the first column pairs' fragments (in the full pass pair 0
        // was loaded before the hand-over into this chunk)
        // (the split-local pass has no outputs: B^T only)
        auto load_pair = [&](int m) __attribute__((always_inline)) {
            if constexpr (kVar || LOCAL) load_bt_of(c, m);
            else load_pair_of(c, m, Irow);
        };
#pragma unroll
        for (int m = LOCAL ? 0 : 1; m < PD && m < NP; ++m) load_pair(m);

        // ---- 2. state projection Y^T = h^T C^T (the Horner steps below
        // give it the decay from the chunk start to the row tile)
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
            }
        }
        state_zero = false;

        // ---- 3. 32-token column pairs, first to last: Horner steps of the
        // chunk state (every pair) and of the output row tiles (pairs left of
        // their diagonal pair)
        float Tchunk = 1.f;
#pragma unroll
        for (int m = 0; m < NP; ++m) {
            if (m + PD < NP) load_pair(m + PD);
            const int slot = m % NS;
            // consume the pair's fragments here on every path, so that their
            // loads stay where they were issued
#pragma unroll
            for (int it = 0; it < IT; ++it)
                if (!kVar && !LOCAL && !(IT == 2 && it == 0 && m >= NP / 2)) asm volatile("" ::"v"(sfr[slot][it]));
            const float tp = sg.Tp[m];
            Tchunk = __fmul_rn(Tchunk, tp);
            bf16x8 xf[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) xf[pt] = sXs[(m * PT + pt) * 64 + lane];

            // chunk state: h^T <- h^T * Tp_m + B_m^T X''_m
            if (st_valid) {
                bf16x8 xs[PTW];
                if constexpr (Cfg::kAllP) {
#pragma unroll
                    for (int k = 0; k < PTW; ++k) xs[k] = xf[k];
                } else {
#pragma unroll
                    for (int k = 0; k < PTW; ++k) xs[k] = sXs[(m * PT + pt0 + k) * 64 + lane];
                }
                // without the output steps in between (the split-local pass,
                // the mask variants), the previous pair's state MFMAs are only
                // a few instructions back
                if constexpr (LOCAL || kVar) mfma_fence_all(hs);
#pragma unroll
                for (int q = 0; q < NTW; ++q) {
#pragma unroll
                    for (int k = 0; k < PTW; ++k) {
                        hs[q * PTW + k] *= tp;
                        hs[q * PTW + k] = mfma_bf16(bfr[slot][q], xs[k], hs[q * PTW + k]);
                    }
                }
            }

            // output rows: Y^T <- Y^T * Tp_m + X''_m^T (C B^T)_{I,m}^T
            if (full && !kVar) {
                // the previous pair's output MFMAs may be only a branch away
                // (ROCm 7.2 has been seen to miss the wait on that path)
                if (m > 0) mfma_fence_all(acc);
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    // statically known: with two row tiles per wave, tile 0
                    // never reaches the upper half of the pairs and tile 1 lies
                    // wholly right of the lower half
                    if (IT == 2 && it == 0 && m >= NP / 2) continue;
                    const bool left = (IT == 2 && it == 1 && m < NP / 2) || m < (Irow[it] >> 1);
                    if (!left) continue;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        acc[it][pt] *= tp;
                        acc[it][pt] = mfma_bf16(xf[pt], sfr[slot][it], acc[it][pt]);
                    }
                }
            }
        }
        split_decay = __fmul_rn(split_decay, Tchunk);

        // ---- 4'. mask variants, per row tile: the row factor on the state
        // projection, then the blocks (I, m), m = I/2 down to 0, each masked
        // element by element and multiplied with the unscaled X of pair m
        if constexpr (kVar) {
            if (full) {
                const bf16x8 *Sc = Sws + (int64_t)c * NBLK * 64;
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int I = Irow[it], I0 = I * 16, i = I0 + l16;
                    const int md = I >> 1;
                    const int rs = resets ? seg_last_reset<Q>(sg, i, I) : -1;
                    const int blk0 = CbShape<Q>::off(I);
                    bf16x8 snext = Sc[(blk0 + md) * 64];
                    // decay from the chunk start through i: the pair decays
                    // left of the diagonal pair, Tb_{I-1} for odd I, F_i
                    float dd[16];
#pragma unroll
                    for (int k = 0; k < 16; k += 4) {
                        const f32x4 v = *(const f32x4 *)&sg.d[I0 + k];
#pragma unroll
                        for (int r = 0; r < 4; ++r) dd[k + r] = v[r];
                    }
                    float ev[4];
                    const float F0 = seg_chain_start(seg_diag_row_regs(dd, I0, i, g, ev), I0, rs);
                    float V = 1.f;
                    for (int mm = 0; mm < md; ++mm) V = __fmul_rn(V, sg.Tp[mm]);
                    if (I & 1) V = __fmul_rn(V, sg.Tb[I - 1]);
                    const float u = __fmul_rn(V, F0);
                    mfma_fence_all(acc[it]);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[it][pt] *= u;
                    const float csi = (SEG == kSegsumDiff) ? vcs[i] : 0.f;
                    float run = 0.f;   // direct: sum of d over (start of the walk, i]
                    auto block = [&](int m, bf16x8 sv, auto DIAG) __attribute__((always_inline)) {
                        constexpr bool diag = decltype(DIAG)::value;
                        // exponents s_ij of the lane's slots j = 32m + 4g + (e%4) + 16(e/4)
                        float se[8];
                        if constexpr (SEG == kSegsumDirect) {
#pragma unroll
                            for (int q = 7; q >= 0; --q) {
                                const f32x4 dq = *(const f32x4 *)&sg.d[32 * m + 4 * q];
#pragma unroll
                                for (int r = 3; r >= 0; --r) {
                                    const int kk = 4 * q + r;
                                    if ((q & 3) == g) se[r + 4 * (q >> 2)] = run;
                                    if (diag) run = (32 * m + kk <= i) ? __fadd_rn(run, dq[r]) : run;
                                    else run = __fadd_rn(run, dq[r]);
                                }
                            }
                        } else {
                            const f32x4 clo = *(const f32x4 *)&vcs[32 * m + 4 * g];
                            const f32x4 chi = *(const f32x4 *)&vcs[32 * m + 16 + 4 * g];
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                se[r] = __fsub_rn(csi, clo[r]);
                                se[4 + r] = __fsub_rn(csi, chi[r]);
                            }
                        }
                        const f32x4 dlo = *(const f32x4 *)&sg.dt[32 * m + 4 * g];
                        const f32x4 dhi = *(const f32x4 *)&sg.dt[32 * m + 16 + 4 * g];
                        bf16x8 pf;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 32 * m + 4 * g + (e & 3) + 16 * (e >> 2);
                            const float dtj = e < 4 ? dlo[e] : dhi[e - 4];
                            const bool zero = (diag && j > i) || j < rs;
                            const float v = zero ? 0.f : __fmul_rn(__builtin_amdgcn_exp2f(se[e]), dtj);
                            pf[e] = (bf16)fmaf((float)sv[e], v, (diag && j == i) ? D_h : 0.f);
                        }
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt)
                            acc[it][pt] = mfma_bf16(sXr[(m * PT + pt) * 64 + lane], pf, acc[it][pt]);
                    };
                    {
                        const bf16x8 sv = snext;
                        if (md > 0) snext = Sc[(blk0 + md - 1) * 64];
                        block(md, sv, std::true_type{});
                    }
                    for (int m = md - 1; m >= 0; --m) {
                        const bf16x8 sv = snext;
                        if (m > 0) snext = Sc[(blk0 + m - 1) * 64];
                        block(m, sv, std::false_type{});
                    }
                }
            }
        }

        // ---- 4. per row tile: the row factor, then the diagonal pair
        //   F_i    decay from the start of row i's sub-block through i
        //   fdg    diagonal-sub-block factor L_ij dt_j
        if (full && !kVar) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int I = Irow[it], I0 = I * 16, i = I0 + l16;
                const int md = I >> 1;
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
                const float Gi = (I & 1) ? __fmul_rn(F0, sg.Tb[max(I - 1, 0)]) : F0;
                const f32x4 dtj = *(const f32x4 *)&sg.dt[I0 + 4 * g];
                float fdg[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = I0 + 4 * g + r;
                    fdg[r] = __fmul_rn(seg_diag_value(ev[r], i, j, rs), dtj[r]);
                }
                // the diagonal pair's C B^T fragment is the row tile's last load
                const int last = (IT == 2 && it == 0) ? NP / 2 - 1 : NP - 1;
                const bf16x8 sv = sfr[last % NS][it];
                bf16x8 pf;
                if (I & 1) {
                    // slots 0..3: sub-block I-1 (L_ij dt_j = F_i W_j dt_j); 4..7: diagonal
                    const f32x4 wlo = *(const f32x4 *)&sg.wd[32 * md + 4 * g];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pf[r] = (bf16)((float)sv[r] * __fmul_rn(F0, wlo[r]));
                        pf[4 + r] = (bf16)fmaf((float)sv[4 + r], fdg[r], (4 * g + r == l16) ? D_h : 0.f);
                    }
                } else {
                    // slots 0..3: diagonal; 4..7: above the diagonal
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pf[r] = (bf16)fmaf((float)sv[r], fdg[r], (4 * g + r == l16) ? D_h : 0.f);
                        pf[4 + r] = (bf16)0.f;
                    }
                }
                mfma_fence_all(acc[it]);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const bf16x8 xr = sXr[(md * PT + pt) * 64 + lane];
                    acc[it][pt] = mfma_bf16(xr, pf, acc[it][pt] * Gi);
                }
            }
        }

        // ---- 5. hand over to the next chunk: after the loads of X_{c+1}
        // have landed, every wave is done with this chunk's fragments and h
        // tile and the producer with y_{c-1}: y_c to the producer, the next
        // fragments and h_c.  The next chunk's C rows go out last: the
        // barrier lets them stay in flight.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (LOCAL) {
            vmem_lds_sync();
        } else {
            // slot 0 takes the next chunk's pair 0: the diagonal pairs (the
            // last loads of each row tile) were read from their slots above
            static_assert(NS >= 2, "pair 0 of the next chunk goes to slot 0");
            load_pair0(cn, Irow);
            load_c(cn, Irow);
            vmem_lds_sync_keep<IT * KN + kPair0Loads>();
        }
        if (full) write_y(Irow);
        if (c + 1 < c_end) {
            mfma_fence_all(hs);
            write_h();
            make_cs(segbuf[buf ^ 1]);
            make_fragments(segbuf[buf ^ 1], c + 1);
        }
        lds_sync();
    }

    // ---- split end: final states (last split) or the split's local summary
    if (!st_valid) return;
    float *dst = nullptr;
    if (full) {
        if (s == a.nsplits - 1 && a.final_states) dst = a.final_states + ((int64_t)b * H + h) * P * N;
    } else {
        dst = a.ws_states + (((int64_t)b * H + h) * a.nsplits + s) * P * N;
        if (tid == 0 && pb == 0 && un.half <= 0) a.ws_decay[((int64_t)b * H + h) * a.nsplits + s] = split_decay;
    }
    if (dst) {
        mfma_fence_all(hs);
        // the lane's row and column are recomputed here from a fresh lane
        // index: the offsets of the entering-state loads are the same, and
        // kept live across the chunk loop they (or the thread index) were
        // spilled to scratch memory
        int le;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(le));
        const int pl = le & 15, nl = 4 * (le >> 4);
#pragma unroll
        for (int k = 0; k < ST; ++k) {
            const int nt = nt0 + k / PTW, pt = pt0 + k % PTW;
            const int p = p_base + pt * 16 + pl, n = nt * 16 + nl;
            *(f32x4 *)(dst + (int64_t)p * N + n) = hs[k];
        }
    }
}

// The head kernel: one workgroup per unit (HALF = false; grid = units -
// half_units) or per half unit of the last, partial round (HALF = true; grid
// = 2 half_units, launched after the first), for the full pass or the
// split-local one.  Each (pass, HALF) is a kernel of its own: one function
// holding several instantiations of the walk kept far more scalar values live
// (measured: 90 scalar registers spilled to vector lanes, 21 without the
// half-unit walk beside the whole-unit one).  sXstage is written only by the
// producer waves' asynchronous loads and read only between the two barriers
// of a hand-over; the fragment sets sXr (unscaled) and sXs (X'') are separate
// LDS objects, so that the compiler sees that their reads do not wait for the
// loads in flight.  sY holds the y tile of one chunk (swizzled like the X
// stage).
//
// SEG != kSegsumHierarchy: the segsum ablation's mask variants (full pass,
// chunk 256); the diff segsum keeps its prefix sums in one more LDS array.
template <int Q, int N, int PB, bool LOCAL, bool HALF, int SEG = kSegsumHierarchy>
__global__ __launch_bounds__(64 * (((Q == 256) ? 8 + SSD_NPROD_Q256 : 4 + 2))) void ssd_scan_bf16_kernel(ChunkArgs a) {
    using Cfg = ScanCfg<Q, N, PB>;
    __shared__ __attribute__((aligned(1024))) bf16 sXstage[Cfg::SX];
    __shared__ __attribute__((aligned(1024))) bf16x8 sXr[Cfg::NFRAG * 64];
    __shared__ __attribute__((aligned(1024))) bf16x8 sXs[Cfg::NFRAG * 64];
    __shared__ __attribute__((aligned(1024))) bf16 sY[Cfg::SX];
    __shared__ __attribute__((aligned(16))) bf16 sH[PB * Cfg::LDH];
    __shared__ __attribute__((aligned(16))) SegBuf<Q> segbuf[2];
    __shared__ __attribute__((aligned(1024))) bf16x8 sTouch[64];   // target of the L2 prefetches
    float *vcs = nullptr;
    if constexpr (SEG == kSegsumDiff) {
        __shared__ __attribute__((aligned(16))) float sCs[Q];
        vcs = sCs;
    }
    if constexpr (HALF) {
        static_assert(PB >= 32, "half units need a headdim block of at least 32");
        const Unit un = unit_of_block(a, a.units - a.half_units + (int)blockIdx.x);
        scan_body<Q, N, PB / 2, LOCAL, SEG>(a, un, un.pb * PB + un.half * (PB / 2), sXstage, sXr, sXs, sY, sH,
                                            segbuf, sTouch, vcs);
    } else {
        const Unit un = unit_of_block(a, (int)blockIdx.x);
        scan_body<Q, N, PB, LOCAL, SEG>(a, un, un.pb * PB, sXstage, sXr, sXs, sY, sH, segbuf, sTouch, vcs);
    }
}

// Launches of one pass (a.mode): the whole units, then the half units.  With
// SEG (a mask variant) only the full pass: the split-local pass has no
// outputs, so the hierarchy kernels serve all three (the caller launches
// them), and each kernel is instantiated in one translation unit only.
template <int Q, int N, int PB, int SEG = kSegsumHierarchy>
inline bool launch_scan_bf16(const ChunkArgs &a, hipStream_t stream) {
    const dim3 block(ScanCfg<Q, N, PB>::THREADS);
    const unsigned whole = (unsigned)(a.units - a.half_units);
    const bool local = a.mode == kModeSplitLocal;
    if (SEG != kSegsumHierarchy && local) return false;
    if (whole > 0) {
        if constexpr (SEG == kSegsumHierarchy) {
            if (local) hipLaunchKernelGGL((ssd_scan_bf16_kernel<Q, N, PB, true, false>), dim3(whole), block, 0, stream, a);
        }
        if (!local) hipLaunchKernelGGL((ssd_scan_bf16_kernel<Q, N, PB, false, false, SEG>), dim3(whole), block, 0, stream, a);
    }
    if constexpr (PB >= 32) {
        if (a.half_units > 0) {
            const dim3 grid((unsigned)(2 * a.half_units));
            if constexpr (SEG == kSegsumHierarchy) {
                if (local) hipLaunchKernelGGL((ssd_scan_bf16_kernel<Q, N, PB, true, true>), grid, block, 0, stream, a);
            }
            if (!local) hipLaunchKernelGGL((ssd_scan_bf16_kernel<Q, N, PB, false, true, SEG>), grid, block, 0, stream, a);
        }
    }
    return true;
}

}  // namespace ssd
