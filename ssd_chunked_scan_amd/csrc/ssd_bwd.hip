// Backward pass of the SSD forward pass (gradients of every input), chunk by
// chunk in reverse, every product on 16x16 MFMA tiles with fp32 accumulation.
//
// With the chunk-entering states H_{c-1} (written by ssd_bwd_states_kernel
// below, one pass over the chunks in order per (batch row, head)) and the
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
// mask is built as the forward kernels build it (nested sums inside 16-token
// sub-blocks, rank-one factors across them).  One workgroup per (batch row,
// head) walks the chunks; dB and dC are written per head and summed over the
// heads of a group by ssd_bwd_reduce_kernel, as are dA and dD over rows.
#include "ssd_common.hpp"
#include "ssd_segsum.hpp"

#include <type_traits>

namespace ssd {

// Element `off` of a row base: the offset is unsigned and 32-bit, so the
// load takes the base in scalar registers and one offset register.
template <typename T>
__device__ inline const T *at_off(const T *p, unsigned off) {
    return (const T *)((const char *)p + off * (unsigned)sizeof(T));
}
__device__ inline float ld1(const float *p, unsigned off) { return *at_off(p, off); }
__device__ inline float ld1(const bf16 *p, unsigned off) { return (float)*at_off(p, off); }

// Four consecutive elements (16-byte fp32 or 8-byte bf16 load), kept packed
// until the MFMA steps take them one by one.
template <typename IO>
struct Pack;
template <>
struct Pack<float> {
    float4 v;
};
template <>
struct Pack<bf16> {
    uint2 v;
};
template <typename IO>
__device__ inline Pack<IO> ld_pack(const IO *p, unsigned off) {
    return Pack<IO>{*(const decltype(Pack<IO>::v) *)at_off(p, off)};
}
template <int E>
__device__ inline float pack_el(const Pack<float> &q) {
    return E == 0 ? q.v.x : E == 1 ? q.v.y : E == 2 ? q.v.z : q.v.w;
}
template <int E>
__device__ inline float pack_el(const Pack<bf16> &q) {
    const unsigned w = (E < 2) ? q.v.x : q.v.y;
    return __uint_as_float((E & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Cross-lane sums and scans on DPP (vector ALU, no LDS round trip).
template <int CTRL>
__device__ inline float dpp_f(float x) {
    return __builtin_bit_cast(float, dpp_row<CTRL>(__builtin_bit_cast(int, x)));
}

// Sum over each row of 16 lanes, every lane receiving it: swaps within pairs
// and quads, then rotations of the row by 4 and by 8.
__device__ inline float row_sum16(float v) {
    v += dpp_f<0xB1>(v);     // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);     // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x124>(v);    // row_ror 4
    return v + dpp_f<0x128>(v);   // row_ror 8
}

// Sum over each aligned group of 8 lanes, every lane receiving it: swaps
// within pairs and quads, then the half-row mirror (lane i and 7 - i).
__device__ inline float group8_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    return v + dpp_f<0x141>(v);   // row_half_mirror
}

// Inclusive prefix sum within each aligned group of 8 lanes; q = lane % 8.
__device__ inline float group8_scan(float v, int q) {
    float o = dpp_f<0x111>(v);    // row_shr 1
    if (q >= 1) v += o;
    o = dpp_f<0x112>(v);          // row_shr 2
    if (q >= 2) v += o;
    o = dpp_f<0x114>(v);          // row_shr 4
    if (q >= 4) v += o;
    return v;
}

// Sum over the whole wave, the same value in every lane: the row sums, then
// lanes 0, 16, 32 and 48 read out and added in a fixed order.
__device__ inline float wave_sum(float v) {
    v = row_sum16(v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// D = A B + C on v_mfma_f32_16x16x4_f32: lane l gives A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 (l / 16) + r][l % 16] in element r.  The
// contraction index of a step is the lane group l / 16; which four values of
// the true index a step covers is free, as long as A and B agree.
__device__ inline f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four steps over the packed elements of a and b (same contraction indices).
template <typename IO>
__device__ inline f32x4 mfma_pack4(const Pack<IO> &a, const Pack<IO> &b, f32x4 c) {
    c = mfma_f32(pack_el<0>(a), pack_el<0>(b), c);
    c = mfma_f32(pack_el<1>(a), pack_el<1>(b), c);
    c = mfma_f32(pack_el<2>(a), pack_el<2>(b), c);
    return mfma_f32(pack_el<3>(a), pack_el<3>(b), c);
}

// Operands of one v_mfma_f32_16x16x32_bf16 step (eight contraction values a
// lane, in the order of eight fp32 steps above): from eight fp32 values,
// rounded to nearest even, or from two packs of four bf16, exact.
__device__ inline bf16x8 bf16x8_of(const float (&v)[8]) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
    return r;
}
__device__ inline bf16x8 bf16x8_of(const Pack<bf16> &lo, const Pack<bf16> &hi) {
    return __builtin_bit_cast(bf16x8, uint4{lo.v.x, lo.v.y, hi.v.x, hi.v.y});
}
// Eight fp32 values as a sum of two bf16 operands: hi = the nearest bf16, lo =
// the nearest bf16 to the remainder.  A product with an exact bf16 operand
// then takes two bf16 steps and keeps about 16 bits of the fp32 value.
__device__ inline void bf16x8_split(const float (&v)[8], bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 h = (bf16)v[e];
        hi[e] = h;
        lo[e] = (bf16)(v[e] - (float)h);
    }
}

// The fp32 MFMA takes more passes than the bf16 one the shared fence is sized
// for: 8 + 4 wait states before vector code reads a result.
__device__ inline void mfma_f32_fence(f32x4 &a, f32x4 &b) {
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(a), "+v"(b));
}

// 8 waves: one workgroup per CU (its LDS allows one), two waves per SIMD
// with 256 registers each; batched operand loads cover the memory latency.
// (16 waves, 128 registers each, measured slower: 6.4 against 6.0 ms at the
// 2.7B layer.)
constexpr int kBwdThreads = 512;

// One instantiation per headdim P (the loops over P have fixed trip counts).
template <typename IO, int P>
__global__ __launch_bounds__(kBwdThreads, 1) void ssd_bwd_kernel(BwdArgs a) {
    constexpr int Q = kBwdQ, NB = Q / 16;
    // Row pitch of the Q x Q matrices: odd, so a lane per row hits its own
    // bank, and 17 mod 64, so the MFMA operand patterns (16 consecutive
    // columns in 4 rows, or 16 rows in 4 consecutive columns) barely collide.
    constexpr int LQ = Q + 17;
    constexpr int kMaxK = 128;              // largest headdim and dstate
    constexpr int kMaxGN = P * (kMaxK + 4);
    constexpr int PU = P / 16;              // 16-column blocks of headdim
    // bf16 inputs: every product of dX, dB, dC and the adjoint update runs on
    // bf16 MFMA with fp32 accumulation.  The masked products take their fp32
    // operand rounded to bf16 (the forward's precision class); the products
    // with the carried states (B G^T, x G, dY H, u dy C^T) take it as hi + lo
    // bf16, two steps, about 16 bits: they give the terms of dl, where sums of
    // both signs magnify rounding.  fp32 inputs keep fp32 MFMA throughout.
    constexpr bool kBf = std::is_same<IO, bf16>::value;
    __shared__ __attribute__((aligned(16))) SegLds<Q> sgb[2];   // segsum values of the chunk (c & 1)
    __shared__ __attribute__((aligned(16))) float sG[kMaxGN];  // adjoint of the state at the chunk end, [P][N + 4]
    // fp32 inputs: the decay mask L[i][j], then V[i][j] = dy_i . x_j, then R's
    // row prefix sums (bf16 inputs form L inside the S/V job instead)
    __shared__ float sL[kBf ? 1 : Q * LQ];
    __shared__ float sS[Q * LQ];            // (L o C B^T)[i][j]
    // fp32 inputs: (L o V)[i][j], the masked operand of dB and dC
    __shared__ float sV[kBf ? 1 : Q * LQ];
    // bf16 inputs: the masked operands of dB and dC as bf16, row t holding
    // (L o V)[i][t] at i (dB) or dt_j (L o V)[t][j] at j (dC), so that a
    // lane group's 8 consecutive tokens (its contraction slots) are one
    // 16-byte read; rows of 64 + 8 elements.  Upper tiles are never written
    // and stay 0 from the clear at the start.
    constexpr int LPB = Q + 8;
    __shared__ __attribute__((aligned(16))) bf16 sLVt[kBf ? Q * LPB : 8], sLdVt[kBf ? Q * LPB : 8];
    // bf16 inputs: the masked operand of dX, (L o S)[.][j] in row j, same layout
    __shared__ __attribute__((aligned(16))) bf16 sLSt[kBf ? Q * LPB : 8];
    __shared__ float swb[2][Q];             // decay from token j to the chunk end (c & 1)
    __shared__ float sq[Q], sp[Q], sxdX[Q], sdl[Q];
    __shared__ float sK, sDD, sDA;
    // Per-wave parts of q, K (one per 16-column block of dstate), p, x . dX
    // (one per 16-column block of headdim) and dy . x (one per wave): each
    // written by one lane, then added in a fixed order, so that every
    // gradient is the same bit for bit from call to call (LDS atomics add in
    // the order the waves arrive).
    __shared__ float sqp[kMaxK / 16][Q], spp[PU][Q], sxdXp[PU][Q];
    __shared__ float sKp[kMaxK / 16], sDDw[kBwdThreads / 64];
    // bf16 inputs with headdim <= 64: the chunk's x, dy, B and C rows are
    // staged in LDS (56 KB), read there by every job.  Row pitches of 40 and
    // 72 dwords (8 mod 32 banks) keep four rows of 16 consecutive columns on
    // distinct banks.
    constexpr bool STAGE = std::is_same<IO, bf16>::value && P <= 64;
    constexpr int XPe = 80, BPe = 144;
    __shared__ __attribute__((aligned(16))) bf16 sXs[STAGE ? Q * XPe : 8], sDYs[STAGE ? Q * XPe : 8];
    __shared__ __attribute__((aligned(16))) bf16 sBs[STAGE ? Q * BPe : 8], sCs[STAGE ? Q * BPe : 8];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: job branches are scalar
    const int L = a.seqlen, H = a.nheads, G = a.ngroups, N = a.dstate;
    const int PN = P * N;
    // The walk: a whole (batch row, head), or one half of a tail walk (chunks
    // [split, nchunks) from dfinal, or [0, split) from the adjoint the states
    // kernel left for it); dA and dD partial sums go to slot 0 or 1
    int bh = blockIdx.x, c_lo = 0, c_hi = a.nchunks, slot = 0;
    const float *g0 = nullptr;
    if (bh >= a.whole_units) {
        const int k = (bh - a.whole_units) >> 1;
        slot = (bh - a.whole_units) & 1;
        bh = a.whole_units + k;
        if (slot == 0)
            c_lo = a.split_chunk;
        else {
            c_hi = a.split_chunk;
            g0 = a.g_tail + (int64_t)k * PN;
        }
    }
    if (slot == 0 && a.dfinal) g0 = a.dfinal + (int64_t)bh * PN;
    const int b = bh / a.nheads, h = bh % a.nheads;
    const int GN = N + 4;                   // row pitch of sG (16-byte rows, 4 mod 64 banks)
    const int grp = h / (H / G);
    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.f;
    const float *dt_row = a.dt + (int64_t)b * L * H + h;
    const int32_t *seq_row = a.seq_idx ? a.seq_idx + (int64_t)b * L : nullptr;
    // element offsets of token t's rows
    auto xo = [&](int t) { return (((int64_t)b * L + t) * H + h) * P; };
    auto bo = [&](int t) { return (((int64_t)b * L + t) * G + grp) * N; };
    const int gxs = H * P, gbs = G * N;     // token strides in global memory
    const int xs = STAGE ? XPe : gxs, bs = STAGE ? BPe : gbs;   // ... where operands are read

    for (int e = tid; e < PN; e += kBwdThreads) sG[(e / N) * GN + e % N] = g0 ? g0[e] : 0.f;
    if constexpr (kBf)
        for (int e = tid; e < Q * LPB / 8; e += kBwdThreads) {
            ((uint4 *)sLVt)[e] = uint4{0u, 0u, 0u, 0u};
            ((uint4 *)sLdVt)[e] = uint4{0u, 0u, 0u, 0u};
            ((uint4 *)sLSt)[e] = uint4{0u, 0u, 0u, 0u};
        }
    if (tid == 0) {
        sDD = 0.f;
        sDA = 0.f;
    }
    if (tid < kBwdThreads / 64) sDDw[tid] = 0.f;
    __syncthreads();

    // The segsum values of a chunk (the forward kernels' helpers) are formed
    // one chunk ahead by the last wave, during the mask phase of the chunk
    // before it in the walk (the mask's row tiles leave that wave idle), into
    // the other of two buffers; the chunk's token values are fetched a chunk
    // before that.
    static_assert(Q == 64 && NB <= kBwdThreads / 64 - 1, "one token a lane; the segsum wave has no mask tile");
    constexpr int SW = kBwdThreads / 64 - 1;   // the segsum wave
    float dt_tok = 0.f;                        // wave SW: token (lane) values fetched ahead
    int flag_tok = 0;
    // The helpers' steps 1-3 in registers (lane = token; a 16-lane DPP row
    // is one sub-block): nested sums by row shifts, in the association order
    // of seg_block_sums' loops (suffix (t, end] from the right, prefix
    // [B0, t] from the left), so every value is the helpers' bit for bit;
    // the sub-block totals and last resets are read out of lanes 16 k and
    // 16 k + 15.  One write of each field.
    auto seg_make = [&](int cc) {   // wave SW only
        const int t = tid & 63, K = t >> 4;
        SegLds<Q> &s = sgb[cc & 1];
        const int flag = flag_tok;
        const float d = __fmul_rn(__fmul_rn(dt_tok, A_h), kLog2e);
        float e = d, pre = d;
#pragma unroll
        for (int k = 0; k < 15; ++k) {
            e = __fadd_rn(dpp_f<kDppRowShl1>(e), d);    // d_t + sum over (t, t + k + 1]
            pre = __fadd_rn(dpp_f<kDppRowShr1>(pre), d);  // sum over [t - k - 1, t]
        }
        const float suf = dpp_f<kDppRowShl1>(e);          // sum over (t, end of sub-block]
        int lastin = -1, fsuf = 0;
        if (seq_row) {
            int v = flag ? t + 1 : 0;                      // 1 + last reset <= t in the sub-block
            v = max(v, dpp_row<kDppRowShr1>(v));
            v = max(v, dpp_row<kDppRowShr1 + 1>(v));
            v = max(v, dpp_row<kDppRowShr1 + 3>(v));
            v = max(v, dpp_row<kDppRowShr1 + 7>(v));
            lastin = v - 1;
            int f = dpp_row<kDppRowShl1>(flag);            // a reset in (t, end of sub-block]
            f |= dpp_row<kDppRowShl1>(f);
            f |= dpp_row<kDppRowShl1 + 1>(f);
            f |= dpp_row<kDppRowShl1 + 3>(f);
            f |= dpp_row<kDppRowShl1 + 7>(f);
            fsuf = f;
        }
        const float W = fsuf ? 0.f : __builtin_amdgcn_exp2f(suf);
        const float u0 = (lastin >= 0) ? 0.f : __builtin_amdgcn_exp2f(pre);
        const float tb = (fsuf | flag) ? 0.f : __builtin_amdgcn_exp2f(e);   // lane 16 k: Tb[k]
        float Tb[NB];
        int blast[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            Tb[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tb), 16 * k));
            blast[k] = __builtin_amdgcn_readlane(lastin, 16 * k + 15);
        }
        const int any = __ballot(flag) != 0ull;
        float V = 1.f, Z = 1.f, T = 1.f;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (k < K) V = __fmul_rn(V, Tb[k]);
            T = __fmul_rn(T, Tb[k]);
        }
#pragma unroll
        for (int k = NB - 1; k >= 0; --k)
            if (k > K) Z = __fmul_rn(Z, Tb[k]);
        int rs = lastin;
        if (any && rs < 0)
#pragma unroll
            for (int k = 0; k < NB; ++k)
                if (k < K && blast[k] >= 0) rs = blast[k];
        s.d[t] = d;
        s.dt[t] = dt_tok;
        s.flag[t] = flag;
        s.W[t] = W;
        s.u[t] = __fmul_rn(u0, V);
        s.wcd[t] = __fmul_rn(__fmul_rn(W, Z), dt_tok);
        s.rs[t] = rs;
        if (t < NB) {
            s.Tb[t] = Tb[t];
            s.blast[t] = blast[t];
        }
        if (t == 0) {
            s.T = T;
            s.any_reset = any;
        }
        swb[cc & 1][t] = __fmul_rn(W, Z);
    };
    if (wave == SW) {
        const int cl0 = c_hi - 1;
        seg_fetch_token(tid & 63, cl0 * Q, min(Q, L - cl0 * Q), dt_row, H, seq_row, dt_tok, flag_tok);
        seg_make(cl0);
        if (cl0 > c_lo) seg_fetch_token(tid & 63, (cl0 - 1) * Q, Q, dt_row, H, seq_row, dt_tok, flag_tok);
    }
    // H_{c-1}: from the forward's scan, or (a single chunk) the initial state or 0
    auto hs_of = [&](int cc) -> const float * {
        return a.states ? a.states + ((int64_t)bh * a.nchunks + cc) * PN
                        : (a.init_states ? a.init_states + (int64_t)bh * PN : nullptr);
    };
    // A wave keeps one block of 16 state columns over its dB/dC jobs (the
    // block count divides the wave count), so it reads those columns of H
    // once per chunk, and a chunk ahead: the read is issued after the jobs
    // of the chunk before.
    static_assert((kBwdThreads / 64) % 8 == 0, "n-block ownership: the block count divides the wave count");
    float hv[4 * PU];
    auto load_hv = [&](int cc, int l16_, int g_) {
        const float *Hc = hs_of(cc);
        const int n = (wave % (N / 16)) * 16 + l16_;
#pragma unroll
        for (int u = 0; u < PU; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                hv[4 * u + e] = Hc ? *at_off(Hc, (16 * u + 4 * g_ + e) * N + n) : 0.f;
    };
    load_hv(c_hi - 1, tid & 15, (tid & 63) >> 4);
    // Staging payload of a chunk, 16 bytes a piece, loaded a chunk ahead into
    // registers (rows past the end of the row hold the last valid token): one
    // piece of x and of dy (Q * P / 8 <= 512 pieces at headdim <= 64) and two
    // of B and of C (Q * N / 8 <= 1024) per thread.  Named registers, not
    // arrays: arrays held across the chunk loop were placed in scratch memory.
    static_assert(!STAGE || (Q * (P / 8) <= kBwdThreads && Q * 16 <= 2 * kBwdThreads),
                  "staging pieces per thread");
    uint4 stx0 = {}, sty0 = {}, stb0 = {}, stb1 = {}, stc0 = {}, stc1 = {};
    auto stage_load = [&](int cc) {
        const int t0c = cc * Q, nv = min(Q, L - t0c);
        if (tid < Q * (P / 8)) {
            const int t = t0c + min(tid / (P / 8), nv - 1), q8 = tid % (P / 8);
            stx0 = *(const uint4 *)((const bf16 *)a.x + xo(t) + q8 * 8);
            sty0 = *(const uint4 *)((const bf16 *)a.dy + xo(t) + q8 * 8);
        }
        const int nb8 = N / 8;
        if (tid < Q * nb8) {
            const int t = t0c + min(tid / nb8, nv - 1), q8 = tid % nb8;
            stb0 = *(const uint4 *)((const bf16 *)a.B + bo(t) + q8 * 8);
            stc0 = *(const uint4 *)((const bf16 *)a.C + bo(t) + q8 * 8);
        }
        if (tid + kBwdThreads < Q * nb8) {
            const int e = tid + kBwdThreads;
            const int t = t0c + min(e / nb8, nv - 1), q8 = e % nb8;
            stb1 = *(const uint4 *)((const bf16 *)a.B + bo(t) + q8 * 8);
            stc1 = *(const uint4 *)((const bf16 *)a.C + bo(t) + q8 * 8);
        }
    };
    auto stage_store = [&]() {
        if (tid < Q * (P / 8)) {
            const int r = tid / (P / 8), q8 = tid % (P / 8);
            *(uint4 *)&sXs[r * XPe + q8 * 8] = stx0;
            *(uint4 *)&sDYs[r * XPe + q8 * 8] = sty0;
        }
        const int nb8 = N / 8;
        if (tid < Q * nb8) {
            const int r = tid / nb8, q8 = tid % nb8;
            *(uint4 *)&sBs[r * BPe + q8 * 8] = stb0;
            *(uint4 *)&sCs[r * BPe + q8 * 8] = stc0;
        }
        if (tid + kBwdThreads < Q * nb8) {
            const int e = tid + kBwdThreads;
            const int r = e / nb8, q8 = e % nb8;
            *(uint4 *)&sBs[r * BPe + q8 * 8] = stb1;
            *(uint4 *)&sCs[r * BPe + q8 * 8] = stc1;
        }
    };
    if constexpr (STAGE) stage_load(c_hi - 1);
    for (int c = c_hi - 1; c >= c_lo; --c) {
        SegLds<Q> &sg = sgb[c & 1];
        float *const sw = swb[c & 1];
        const int t0 = c * Q;
        const int nvalid = min(Q, L - t0);
        const float *Hs = hs_of(c);
        // operand row of token t0 + t, or none past the end of the row
        auto ok = [&](int t) { return t < nvalid; };
        // The lane index, opaque to the compiler here: the per-lane offsets
        // of the unrolled operand loads are recomputed per chunk rather than
        // hoisted out of the loop and kept live (they would spill).
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));
        const int l16 = lane & 15, g = lane >> 4;
        // Operand rows past the end of the row are read at the last valid
        // token instead: every product they enter is zeroed by the mask, by
        // dt = 0, or by the output row's own guard (the state update zeroes
        // them explicitly).
        auto cl = [&](int t) { return min(t, nvalid - 1); };
        // Contraction slots of the masked products and the adjoint update
        // with bf16 inputs: lane group g takes the 8 consecutive tokens
        // 32 q + 8 g + e of slab q (fp32 inputs: token 4 st + g of step st).
        // With staged rows a column's 8 tokens are two 16-bit transpose reads
        // of four consecutive rows (rows past the end hold the last valid
        // token; every product meets a 0 there).
        auto ktok = [&](int st) { return kBf ? 32 * (st >> 3) + 8 * g + (st & 7) : 4 * st + g; };
        auto tr8 = [&](const bf16 *base, int pitch, int q, int col0) {
            const int rr = 32 * q + 8 * g + (l16 >> 2), cc = col0 + 4 * (l16 & 3);
            return join_bf16x8(lds_read_tr16(base + rr * pitch + cc), lds_read_tr16(base + (rr + 4) * pitch + cc));
        };
        // the chunk's first token rows; tokens step by xs (x, dy) or bs (B, C)
        // elements, so in-chunk offsets fit 32 bits and the loads take a
        // scalar base
        const IO *xc, *dyc, *Bc, *Cc;
        if constexpr (STAGE) {
            // the previous chunk's last reads of the staged rows are behind
            // its final barrier
            stage_store();
            xc = (const IO *)sXs;
            dyc = (const IO *)sDYs;
            Bc = (const IO *)sBs;
            Cc = (const IO *)sCs;
        } else {
            xc = (const IO *)a.x + xo(t0);
            dyc = (const IO *)a.dy + xo(t0);
            Bc = (const IO *)a.B + bo(t0);
            Cc = (const IO *)a.C + bo(t0);
        }

        // the chunk's segsum values are in sgb[c & 1] (formed during the
        // previous chunk, or before the walk); this barrier also publishes
        // the staged rows and the cleared per-chunk sums
        for (int e = tid; e < (kMaxK / 16) * Q; e += kBwdThreads) (&sqp[0][0])[e] = 0.f;
        for (int e = tid; e < PU * Q; e += kBwdThreads) {
            (&spp[0][0])[e] = 0.f;
            (&sxdXp[0][0])[e] = 0.f;
        }
        if (tid < kMaxK / 16) sKp[tid] = 0.f;
        __syncthreads();

        // the segsum wave: the next chunk's values (chunk c - 1, whole), then
        // the fetch of the chunk after it; its buffer was the previous chunk's,
        // whose readers are behind the barriers since.  It runs in the first
        // phase that leaves it idle: the mask (fp32 inputs), or the S/V jobs
        // (bf16 inputs: ten jobs over eight waves).
        auto seg_ahead = [&] {
            if (wave == SW && c > c_lo) {
                seg_make(c - 1);
                if (c - 1 > c_lo) seg_fetch_token(tid & 63, (c - 2) * Q, Q, dt_row, H, seq_row, dt_tok, flag_tok);
            }
        };

        // ---- mask (fp32 inputs), built as the forward kernels build it:
        // nested sums inside 16-token sub-blocks, rank-one factors across them.
        // A wave takes a 16-row tile, a lane row i and columns 16 jt + 4 g + r.
        if constexpr (!kBf) {
        for (int I = wave; I < NB; I += kBwdThreads / 64) {
            const int i = I * 16 + l16;
            const int rs_i = sg.rs[i];
            float e[4];
            const float sum0 = seg_diag_row(sg.d, I * 16, i, g, e);
            float F = seg_chain_start(sum0, I * 16, rs_i);
            for (int jt = NB - 1; jt >= 0; --jt) {
                float v[4] = {0.f, 0.f, 0.f, 0.f};
                if (jt == I) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = seg_diag_value(e[r], i, jt * 16 + 4 * g + r, rs_i);
                } else if (jt < I) {
                    if (jt < I - 1) F = seg_chain_step(F, sg.Tb[jt + 1]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = seg_offdiag(F, sg.W[jt * 16 + 4 * g + r]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sL[i * LQ + jt * 16 + 4 * g + r] = (i < nvalid) ? v[r] : 0.f;
            }
        }
        seg_ahead();
        __syncthreads();
        }

        // ---- S = C B^T and V = dY X^T on the lower 16 x 16 tiles (upper tiles
        // are never read), one job per tile computing both.  Stored: L o S in
        // sS, L o V in sV (what dX, dB and dC read), and V itself over L in
        // sL (only the R walk reads it; L is not read again in the chunk).
        // Both operands are rows of token-major arrays: a lane reads
        // consecutive elements of its row and feeds them to its steps; all
        // loads of a product are issued before its MFMAs.
        {
            auto product = [&](const IO *Ab, const IO *Bb, unsigned ao, unsigned bo_, int K)
                    __attribute__((always_inline)) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
                if constexpr (STAGE) {
                    // bf16 rows in LDS: v_mfma_f32_16x16x32_bf16, a lane
                    // giving eight consecutive elements of its row (products
                    // of bf16 values are exact, accumulation fp32 as above)
#pragma unroll
                    for (int u = 0; u < kMaxK / 32; u += 2) {
                        if (32 * u + 32 > K) break;   // whole 32-wide steps only (K = 16: the half step below)
                        const bf16x8 a0 = *(const bf16x8 *)at_off(Ab, ao + 32 * u + 8 * g);
                        const bf16x8 b0 = *(const bf16x8 *)at_off(Bb, bo_ + 32 * u + 8 * g);
                        acc = mfma_bf16(a0, b0, acc);
                        if (32 * (u + 1) + 32 <= K) {
                            const bf16x8 a1 = *(const bf16x8 *)at_off(Ab, ao + 32 * (u + 1) + 8 * g);
                            const bf16x8 b1 = *(const bf16x8 *)at_off(Bb, bo_ + 32 * (u + 1) + 8 * g);
                            acc2 = mfma_bf16(a1, b1, acc2);
                        }
                    }
                    if (K == 16) {   // a half step: the upper eight of the 32 contraction slots are 0
                        const bf16x8 z = {};
                        const bf16x8 a0 = g < 2 ? *(const bf16x8 *)at_off(Ab, ao + 8 * g) : z;
                        const bf16x8 b0 = g < 2 ? *(const bf16x8 *)at_off(Bb, bo_ + 8 * g) : z;
                        acc = mfma_bf16(a0, b0, acc);
                    }
                } else {
                    Pack<IO> av[kMaxK / 16], bv[kMaxK / 16];
#pragma unroll
                    for (int u = 0; u < kMaxK / 16; ++u) {
                        const bool in = 16 * u < K;
                        av[u] = in ? ld_pack<IO>(Ab, ao + 16 * u + 4 * g) : Pack<IO>{};
                        bv[u] = in ? ld_pack<IO>(Bb, bo_ + 16 * u + 4 * g) : Pack<IO>{};
                    }
#pragma unroll
                    for (int u = 0; u < kMaxK / 16; u += 2) {
                        if (16 * u >= K) break;
                        acc = mfma_pack4(av[u], bv[u], acc);
                        acc2 = mfma_pack4(av[u + 1], bv[u + 1], acc2);
                    }
                }
                mfma_f32_fence(acc, acc2);
                return f32x4{acc[0] + acc2[0], acc[1] + acc2[1], acc[2] + acc2[2], acc[3] + acc2[3]};
            };
            constexpr int NT = NB * (NB + 1) / 2;
            for (int job = wave; job < NT; job += kBwdThreads / 64) {
                int k = job, I = 0;
                while (k > I) k -= ++I;
                const int J = k;                              // tile (I, J), J <= I
                const int i = I * 16 + l16, j = J * 16 + l16;
                const f32x4 sv = product(Cc, Bc, cl(i) * bs, cl(j) * bs, N);
                const f32x4 vv = product(dyc, xc, cl(i) * xs, cl(j) * xs, P);
                if constexpr (kBf) {
                    // the mask entries of this lane, L[ii][j] for rows
                    // ii = 16 I + 4 g + r, with the mask loop's arithmetic:
                    // diagonal tile, the nested sum over (j, ii] added from ii
                    // down; off the diagonal, the chain start (the sum over
                    // [16 I, ii]) times the sub-block decays Tb[I-1] .. Tb[J+1]
                    // in that order, times W_j
                    const int I0 = I * 16;
                    float dd[16];
#pragma unroll
                    for (int kk = 0; kk < 16; ++kk) dd[kk] = sg.d[I0 + kk];
                    const float dtj = sg.dt[j], Wj = sg.W[j];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ii = I0 + 4 * g + r;
                        const int rs_i = sg.rs[ii];
                        float lm;
                        if (I == J) {
                            float es = 0.f;
#pragma unroll
                            for (int kk = 15; kk >= 0; --kk)
                                if (I0 + kk <= ii && I0 + kk > j) es = __fadd_rn(es, dd[kk]);
                            lm = seg_diag_value(es, ii, j, rs_i);
                        } else {
                            float sum0 = 0.f;
#pragma unroll
                            for (int kk = 15; kk >= 0; --kk)
                                if (I0 + kk <= ii) sum0 = __fadd_rn(sum0, dd[kk]);
                            float F = seg_chain_start(sum0, I0, rs_i);
                            for (int jt = I - 2; jt >= J; --jt) F = seg_chain_step(F, sg.Tb[jt + 1]);
                            lm = seg_offdiag(F, Wj);
                        }
                        if (ii >= nvalid) lm = 0.f;
                        const float ls = lm * sv[r], lv = lm * vv[r];
                        // (L o S)[ii][j] and (L o V)[ii][j] into row j of the dX
                        // and dB operands at token ii; dt_j (L o V)[ii][j] into
                        // row ii of the dC operand at token j; R[ii][j] =
                        // (L o S) dt V (the order of the fp32 path's R walk)
                        sLSt[j * LPB + ii] = (bf16)ls;
                        sLVt[j * LPB + ii] = (bf16)lv;
                        sLdVt[ii * LPB + j] = (bf16)(dtj * lv);
                        sS[ii * LQ + j] = ls * dtj * vv[r];
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = (I * 16 + 4 * g + r) * LQ + J * 16 + l16;
                        const float l = sL[e];
                        sS[e] = l * sv[r];
                        sV[e] = l * vv[r];
                        sL[e] = vv[r];
                    }
                }
            }
        }
        if constexpr (kBf) seg_ahead();
        __syncthreads();

        float ddsum = 0.f;
        // ---- dX (and x . dX, p_r), dx, and dy . x for dD: tiles over (j, p)
        //   acc  = sum_{i >= j} (L o S)[i][j] dy_i[p]     (i: LDS column, dy rows)
        //   acc2 = (B G^T)[j][p] = G B_j                  (n: B rows, G rows)
        // A wave takes one block of 16 headdim columns p and NJ consecutive
        // 16-row blocks J of it; dy's columns and G's rows for p are read once
        // for all of them.  Steps above a tile's triangle are removed by a
        // select (upper tiles of S are never written).
        {
            const int NJ = max(1, PU / 2);
            const int Pb = wave % PU, J0 = (wave / PU) * NJ;
            const int p = Pb * 16 + l16;
            if (J0 < NB) {
                float dyv[4 * NB];
                float4 gv[kMaxK / 16];
#pragma unroll
                for (int st = 0; st < 4 * NB; ++st)
                    dyv[st] = STAGE ? 0.f : ld1(dyc, cl(ktok(st)) * xs + p);   // staged: transpose reads below
#pragma unroll
                for (int u = 0; u < kMaxK / 16; ++u)   // blocks past N: B is 0 there, G read at a valid column
                    gv[u] = *(const float4 *)&sG[p * GN + min(16 * u, N - 16) + 4 * g];
                bf16x8 ghi[kMaxK / 32], glo[kMaxK / 32];
                if constexpr (kBf) {
#pragma unroll
                    for (int v = 0; v < kMaxK / 32; ++v) {
                        const float w[8] = {gv[2 * v].x, gv[2 * v].y, gv[2 * v].z, gv[2 * v].w,
                                            gv[2 * v + 1].x, gv[2 * v + 1].y, gv[2 * v + 1].z, gv[2 * v + 1].w};
                        bf16x8_split(w, ghi[v], glo[v]);
                    }
                }
                for (int J = J0; J < J0 + NJ; ++J) {
                    const int jr = J * 16 + l16;
                    const unsigned brow = cl(jr) * bs;
                    Pack<IO> bv[kMaxK / 16];
#pragma unroll
                    for (int u = 0; u < kMaxK / 16; ++u)
                        bv[u] = (16 * u < N) ? ld_pack<IO>(Bc, brow + 16 * u + 4 * g) : Pack<IO>{};
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
                    // i = 16 J .. Q - 1: whole 16-row blocks I >= J (one uniform
                    // branch per block; inside the diagonal block L is 0 above
                    // the diagonal)
                    if constexpr (kBf) {
                        // one bf16 step per two 16-row blocks (slot e in block
                        // 2q + e/4; a block left of J is zeroed)
#pragma unroll
                        for (int q = 0; q < NB / 2; ++q) {
                            if (2 * q + 1 < J) continue;
                            bf16x8 bb;
                            if constexpr (STAGE) {
                                bb = tr8(sDYs, XPe, q, Pb * 16);
                            } else {
                                float bw[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) bw[e] = dyv[8 * q + e];
                                bb = bf16x8_of(bw);
                            }
                            const bf16x8 av = *(const bf16x8 *)&sLSt[jr * LPB + 32 * q + 8 * g];   // (L o S)[i][j]
                            acc = mfma_bf16(av, bb, acc);
                        }
                    } else {
#pragma unroll
                        for (int blk = 0; blk < NB; ++blk) {
                            if (blk < J) continue;
#pragma unroll
                            for (int s4 = 0; s4 < 4; ++s4) {
                                const int st = 4 * blk + s4;
                                acc = mfma_f32(sS[(4 * st + g) * LQ + jr], dyv[st], acc);
                            }
                        }
                    }
                    // B G^T also gives p_r, a term of dl, where sums of both
                    // signs magnify operand rounding (G rounded to bf16: dA
                    // 1.5e-2 off at headdim 16): G as hi + lo bf16
                    if constexpr (kBf) {
#pragma unroll
                        for (int v = 0; v < kMaxK / 32; ++v) {
                            if (32 * v >= N) break;
                            const bf16x8 bb = bf16x8_of(bv[2 * v], bv[2 * v + 1]);
                            acc2 = mfma_bf16(bb, ghi[v], acc2);
                            acc2 = mfma_bf16(bb, glo[v], acc2);
                        }
                    } else {
#pragma unroll
                        for (int u = 0; u < kMaxK / 16; ++u) {
                            acc2 = mfma_f32(pack_el<0>(bv[u]), gv[u].x, acc2);
                            acc2 = mfma_f32(pack_el<1>(bv[u]), gv[u].y, acc2);
                            acc2 = mfma_f32(pack_el<2>(bv[u]), gv[u].z, acc2);
                            acc2 = mfma_f32(pack_el<3>(bv[u]), gv[u].w, acc2);
                        }
                    }
                    mfma_f32_fence(acc, acc2);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = J * 16 + 4 * g + r;
                        float xd = 0.f, pr = 0.f;
                        if (ok(j)) {
                            const float dX = fmaf(sw[j], acc2[r], acc[r]);
                            const float xv = ld1(xc, j * xs + p);
                            const float dyj = ld1(dyc, j * xs + p);
                            a.dx[xo(t0 + j) + p] = fmaf(sg.dt[j], dX, D_h * dyj);
                            xd = xv * dX;
                            pr = sg.wcd[j] * xv * acc2[r];
                            ddsum = fmaf(dyj, xv, ddsum);
                        }
                        xd = row_sum16(xd);
                        pr = row_sum16(pr);
                        if (l16 == 0 && ok(j)) {
                            sxdXp[Pb][j] = xd;
                            spp[Pb][j] = pr;
                        }
                    }
                }
            }
        }
        // ---- dB, dC (per head) and q_s: tiles over (t, n)
        //   dB: acc = sum_{i >= t} (L o V)[i][t] C_i[n],  acc2 = (X G)[t][n] = G^T x_t
        //   dC: acc = sum_{j <= t} (L o dt o V)[t][j] B_j[n],  acc2 = (dY H)[t][n] = H^T dy_t
        // the first wave on each block of state columns (T0 = 0) adds its
        // share of T <G, H> from the G columns it holds
        // A wave takes one block of 16 state columns n and NT consecutive
        // 16-row blocks T of it (NT = 4 at dstate 128: the whole chunk).  The
        // B operands of those tiles (C and B columns, G columns) are the same
        // for every T and are read once.  Steps outside a tile's triangle are
        // removed by a select (upper tiles of V are never written).
        {
            const int NT = max(1, N / 32);
            const int Nb = wave % (N / 16), T0 = (wave / (N / 16)) * NT;
            const int n = Nb * 16 + l16;
            if (T0 < NB) {
                float cvs[4 * NB], bvs[4 * NB], gq[4 * PU];
#pragma unroll
                for (int st = 0; st < 4 * NB; ++st) {   // staged: transpose reads below
                    const int i = ktok(st);
                    cvs[st] = STAGE ? 0.f : ld1(Cc, cl(i) * bs + n);
                    bvs[st] = STAGE ? 0.f : ld1(Bc, cl(i) * bs + n);
                }
#pragma unroll
                for (int u = 0; u < PU; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) gq[4 * u + e] = sG[(16 * u + 4 * g + e) * GN + n];
                if (Hs && T0 == 0) {
                    float k = 0.f;
#pragma unroll
                    for (int e = 0; e < 4 * PU; ++e) k = fmaf(gq[e], hv[e], k);
                    k = wave_sum(k);
                    if (lane == 0) sKp[Nb] = k;   // T0 == 0: one wave per Nb
                }
                // bf16: G and H columns as hi + lo bf16 (see dX)
                constexpr int PV = (PU + 1) / 2;
                bf16x8 gqhi[PV], gqlo[PV], hvhi[PV], hvlo[PV];
                if constexpr (kBf) {
#pragma unroll
                    for (int v = 0; v < PV; ++v) {
                        float w[8], x8[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const bool in = 8 * v + e < 4 * PU;
                            w[e] = in ? gq[min(8 * v + e, 4 * PU - 1)] : 0.f;
                            x8[e] = in ? hv[min(8 * v + e, 4 * PU - 1)] : 0.f;
                        }
                        bf16x8_split(w, gqhi[v], gqlo[v]);
                        bf16x8_split(x8, hvhi[v], hvlo[v]);
                    }
                }
                for (int T = T0; T < T0 + NT; ++T) {
                    const int tr = T * 16 + l16;
                    const unsigned trow = cl(tr) * xs;
                    Pack<IO> xr[PU], dr[PU];
                    float cq[4];
#pragma unroll
                    for (int u = 0; u < PU; ++u) {
                        xr[u] = ld_pack<IO>(xc, trow + 16 * u + 4 * g);
                        dr[u] = Hs ? ld_pack<IO>(dyc, trow + 16 * u + 4 * g) : Pack<IO>{};
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) cq[r] = ld1(Cc, cl(T * 16 + 4 * g + r) * bs + n);
                    // dB: i = 16 T .. Q - 1;  G^T x_t
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (kBf) {
#pragma unroll
                        for (int q = 0; q < NB / 2; ++q) {   // pairs of blocks; blocks I < T read as 0
                            if (2 * q + 1 < T) continue;
                            bf16x8 bb;
                            if constexpr (STAGE) {
                                bb = tr8(sCs, BPe, q, Nb * 16);
                            } else {
                                float bw[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) bw[e] = cvs[8 * q + e];
                                bb = bf16x8_of(bw);
                            }
                            const bf16x8 av = *(const bf16x8 *)&sLVt[tr * LPB + 32 * q + 8 * g];   // (L o V)[i][t]
                            acc = mfma_bf16(av, bb, acc);
                        }
#pragma unroll
                        for (int v = 0; v < PV; ++v) {
                            const Pack<IO> hi = (2 * v + 1 < PU) ? xr[min(2 * v + 1, PU - 1)] : Pack<IO>{};
                            const bf16x8 xx = bf16x8_of(xr[2 * v], hi);   // x_t, G columns
                            acc2 = mfma_bf16(xx, gqhi[v], acc2);
                            acc2 = mfma_bf16(xx, gqlo[v], acc2);
                        }
                    } else {
#pragma unroll
                        for (int blk = 0; blk < NB; ++blk) {   // whole blocks I >= T
                            if (blk < T) continue;
#pragma unroll
                            for (int s4 = 0; s4 < 4; ++s4) {
                                const int st = 4 * blk + s4;
                                acc = mfma_f32(sV[(4 * st + g) * LQ + tr], cvs[st], acc);   // (L o V)[i][t]
                            }
                        }
#pragma unroll
                        for (int u = 0; u < PU; ++u) {
                            acc2 = mfma_f32(pack_el<0>(xr[u]), gq[4 * u], acc2);
                            acc2 = mfma_f32(pack_el<1>(xr[u]), gq[4 * u + 1], acc2);
                            acc2 = mfma_f32(pack_el<2>(xr[u]), gq[4 * u + 2], acc2);
                            acc2 = mfma_f32(pack_el<3>(xr[u]), gq[4 * u + 3], acc2);
                        }
                    }
                    mfma_f32_fence(acc, acc2);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = T * 16 + 4 * g + r;
                        if (ok(t)) a.dB_head[(((int64_t)b * L + t0 + t) * H + h) * N + n] = sg.dt[t] * fmaf(sw[t], acc2[r], acc[r]);
                    }
                    // dC: j = 0 .. 16 T + 15;  H^T dy_t
                    acc = f32x4{0.f, 0.f, 0.f, 0.f};
                    acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (kBf) {
#pragma unroll
                        for (int q = 0; q < NB / 2; ++q) {   // pairs of blocks; blocks J > T read as 0
                            if (2 * q > T) break;
                            bf16x8 bb;
                            if constexpr (STAGE) {
                                bb = tr8(sBs, BPe, q, Nb * 16);
                            } else {
                                float bw[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) bw[e] = bvs[8 * q + e];
                                bb = bf16x8_of(bw);
                            }
                            const bf16x8 av = *(const bf16x8 *)&sLdVt[tr * LPB + 32 * q + 8 * g];   // (L o dt o V)[t][j]
                            acc = mfma_bf16(av, bb, acc);
                        }
                    } else {
#pragma unroll
                        for (int blk = 0; blk < NB; ++blk) {   // whole blocks J <= T
                            if (blk > T) break;
#pragma unroll
                            for (int s4 = 0; s4 < 4; ++s4) {
                                const int j = 4 * (4 * blk + s4) + g;
                                acc = mfma_f32(sg.dt[j] * sV[tr * LQ + j], bvs[4 * blk + s4], acc);   // (L o dt o V)[t][j]
                            }
                        }
                    }
                    // dY H also gives q_s, a term of dl: H as hi + lo bf16
                    if constexpr (kBf) {
#pragma unroll
                        for (int v = 0; v < PV; ++v) {
                            const Pack<IO> hi = (2 * v + 1 < PU) ? dr[min(2 * v + 1, PU - 1)] : Pack<IO>{};
                            const bf16x8 dd = bf16x8_of(dr[2 * v], hi);   // dy_t, H columns
                            acc2 = mfma_bf16(dd, hvhi[v], acc2);
                            acc2 = mfma_bf16(dd, hvlo[v], acc2);
                        }
                    } else {
#pragma unroll
                        for (int u = 0; u < PU; ++u) {
                            acc2 = mfma_f32(pack_el<0>(dr[u]), hv[4 * u], acc2);
                            acc2 = mfma_f32(pack_el<1>(dr[u]), hv[4 * u + 1], acc2);
                            acc2 = mfma_f32(pack_el<2>(dr[u]), hv[4 * u + 2], acc2);
                            acc2 = mfma_f32(pack_el<3>(dr[u]), hv[4 * u + 3], acc2);
                        }
                    }
                    mfma_f32_fence(acc, acc2);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = T * 16 + 4 * g + r;
                        float qv = 0.f;
                        if (ok(t)) {
                            a.dC_head[(((int64_t)b * L + t0 + t) * H + h) * N + n] = fmaf(sg.u[t], acc2[r], acc[r]);
                            qv = sg.u[t] * acc2[r] * cq[r];
                        }
                        qv = row_sum16(qv);
                        if (l16 == 0 && ok(t)) sqp[Nb][t] = qv;
                    }
                }
            }
        }
        if (c > c_lo) load_hv(c - 1, l16, g);
        ddsum = wave_sum(ddsum);
        if (lane == 0) sDDw[wave] += ddsum;
        __syncthreads();

        // ---- R = L o dt o S o V, then prefix sums of each row over r < t
        // (eight lanes per row, eight columns each)
        constexpr int LPR = kBwdThreads / Q, CPL = Q / LPR;   // lanes per row, columns per lane
        static_assert(LPR * Q == kBwdThreads && LPR == 8, "rows of 8 lanes (the DPP sums and scans)");
        {
            const int s = tid / LPR, q = tid % LPR;
            float Rv[CPL], loc = 0.f;
#pragma unroll
            for (int c8 = 0; c8 < CPL; ++c8) {
                const int r = CPL * q + c8;
                if constexpr (kBf)
                    Rv[c8] = (r <= s) ? sS[s * LQ + r] : 0.f;   // R, formed by the S/V job
                else
                    Rv[c8] = (r <= s) ? sS[s * LQ + r] * sg.dt[r] * sL[s * LQ + r] : 0.f;   // (L o S) dt V
                loc += Rv[c8];
            }
            float run = group8_scan(loc, q) - loc;
#pragma unroll
            for (int c8 = 0; c8 < CPL; ++c8) {
                (kBf ? sS : sL)[s * LQ + CPL * q + c8] = run;   // sum_{r' < r} R_{s r'}, over what was read above
                run += Rv[c8];
            }
            // the per-wave parts of q_s, p_s, x_s . dX_s and K: lane q of the
            // row takes part q (parts past dstate or headdim hold 0), then
            // the row's eight lanes are summed in a fixed order
            static_assert(kMaxK / 16 == LPR && PU <= LPR, "one part per lane of a row");
            const float vq = group8_sum(sqp[q][s]);
            const float vp = group8_sum(q < PU ? spp[q][s] : 0.f);
            const float vx = group8_sum(q < PU ? sxdXp[q][s] : 0.f);
            const float vk = group8_sum(sKp[q]);
            if (q == 0) {
                sq[s] = vq;
                sp[s] = vp;
                sxdX[s] = vx;
                if (s == 0) sK = vk;
            }
        }
        __syncthreads();
        {
            const int t = tid / LPR, q = tid % LPR;
            float dl = 0.f;
#pragma unroll
            for (int k8 = 0; k8 < CPL; ++k8) {
                const int s = q + LPR * k8;
                if (s >= t) dl += (kBf ? sS : sL)[s * LQ + t] + sq[s];
                else dl += sp[s];
            }
            dl = group8_sum(dl);
            if (q == 0) {
                if (t < nvalid) {
                    dl += sg.T * sK;
                    if (sg.flag[t]) dl = 0.f;   // a_t is 0 there, not exp(dt A)
                    a.ddt[((int64_t)b * L + t0 + t) * H + h] = fmaf(A_h, dl, sxdX[t]);
                }
                sdl[t] = (t < nvalid) ? sg.dt[t] * dl : 0.f;
            }
        }
        // The next chunk's rows go into flight here, after this chunk's last
        // global store: vmcnt also counts stores, and the wait for these loads
        // at the next chunk's start then finds nothing younger to drain.
        if constexpr (STAGE)
            if (c > c_lo) stage_load(c - 1);
        // ---- G_{c-1} = T G_c + sum_i u_i dy_i C_i^T: tiles over (p, n)
        // A wave keeps one block of 16 headdim rows p (the block count divides
        // the wave count) over its tiles, so u o dy for those rows is read once.
        {
            constexpr int kWaves = kBwdThreads / 64;
            static_assert(kWaves % 8 == 0, "headdim blocks divide the wave count");
            const int Pb = wave % PU;
            const int p = Pb * 16 + l16;
            if constexpr (STAGE) {
                // staged bf16 rows: the u o dy and C columns by transpose
                // reads, tokens 32 q + 8 g + e (u = 0 past the end)
                bf16x8 dvhi[NB / 2], dvlo[NB / 2];
#pragma unroll
                for (int q = 0; q < NB / 2; ++q) {
                    const bf16x8 d8 = tr8(sDYs, XPe, q, Pb * 16);
                    const float4 u0 = *(const float4 *)&sg.u[32 * q + 8 * g];
                    const float4 u1 = *(const float4 *)&sg.u[32 * q + 8 * g + 4];
                    const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                    float w[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = ok(32 * q + 8 * g + e) ? uu[e] * (float)d8[e] : 0.f;
                    bf16x8_split(w, dvhi[q], dvlo[q]);
                }
                for (int Nb = wave / PU; Nb < N / 16; Nb += kWaves / PU) {
                    const int n = Nb * 16 + l16;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < NB / 2; ++q) {
                        if (32 * q >= nvalid) break;
                        const bf16x8 cc = tr8(sCs, BPe, q, Nb * 16);
                        acc = mfma_bf16(dvhi[q], cc, acc);
                        acc2 = mfma_bf16(dvlo[q], cc, acc2);
                    }
                    mfma_f32_fence(acc, acc2);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float *gp = &sG[(Pb * 16 + 4 * g + r) * GN + n];
                        *gp = fmaf(sg.T, *gp, acc[r] + acc2[r]);
                    }
                }
            } else {
            float dv[4 * NB];
#pragma unroll
            for (int st = 0; st < 4 * NB; ++st) {
                const int i = 4 * st + g;
                dv[st] = (ok(i) ? sg.u[i] : 0.f) * ld1(dyc, cl(i) * xs + p);
            }
            // bf16: u o dy as hi + lo bf16 (G carries into every later chunk's
            // terms of dl), C exact
            bf16x8 dvhi[NB / 2], dvlo[NB / 2];
            if constexpr (kBf) {
#pragma unroll
                for (int q = 0; q < NB / 2; ++q) {
                    float w[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = dv[8 * q + e];
                    bf16x8_split(w, dvhi[q], dvlo[q]);
                }
            }
            for (int Nb = wave / PU; Nb < N / 16; Nb += kWaves / PU) {
                const int n = Nb * 16 + l16;
                float cv[4 * NB];
#pragma unroll
                for (int st = 0; st < 4 * NB; ++st) cv[st] = ld1(Cc, cl(4 * st + g) * bs + n);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
                if constexpr (kBf) {
#pragma unroll
                    for (int q = 0; q < NB / 2; ++q) {
                        if (32 * q >= nvalid) break;
                        float w[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[e] = cv[8 * q + e];
                        const bf16x8 cc = bf16x8_of(w);
                        acc = mfma_bf16(dvhi[q], cc, acc);
                        acc2 = mfma_bf16(dvlo[q], cc, acc2);
                    }
                } else {
#pragma unroll
                    for (int st = 0; st < 4 * NB; st += 2) {
                        if (4 * st >= nvalid) break;
                        acc = mfma_f32(dv[st], cv[st], acc);
                        acc2 = mfma_f32(dv[st + 1], cv[st + 1], acc2);
                    }
                }
                mfma_f32_fence(acc, acc2);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float *gp = &sG[(Pb * 16 + 4 * g + r) * GN + n];
                    *gp = fmaf(sg.T, *gp, acc[r] + acc2[r]);
                }
            }
            }
        }
        __syncthreads();
        static_assert(Q == 64, "one token a lane of wave 0");
        if (tid < 64) {
            const float s = wave_sum(sdl[tid]);
            if (tid == 0) sDA += s;
        }
    }
    __syncthreads();
    if (a.dinit && c_lo == 0)
        for (int e = tid; e < PN; e += kBwdThreads) a.dinit[(int64_t)bh * PN + e] = sG[(e / N) * GN + e % N];
    if (tid == 0) {
#pragma unroll
        for (int w = 0; w < kBwdThreads / 64; ++w) sDD += sDDw[w];
        a.dA_part[2 * bh + slot] = sDA;
        a.dD_part[2 * bh + slot] = sDD;
        if (c_lo == 0 && c_hi == a.nchunks) {   // a whole walk fills both slots
            a.dA_part[2 * bh + 1] = 0.f;
            a.dD_part[2 * bh + 1] = 0.f;
        }
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
            const int64_t o = 2 * ((int64_t)bb * H + h);
            sa += a.dA_part[o];
            sa += a.dA_part[o + 1];
            sd += a.dD_part[o];
            sd += a.dD_part[o + 1];
        }
        a.dA[h] = sa;
        if (a.dD) a.dD[h] = sd;
    }
}

// ---------------------------------------------------------------------------
// The chunk-entering states the reverse walk reads: H_{c-1} for every
// 64-token chunk c, as [batch][nheads][nchunks][headdim][dstate] fp32, entry 0
// being the initial state (or 0).  One workgroup per (batch row, head) walks
// the chunks in order with the state in MFMA accumulators,
//   H_c = T_c H_{c-1} + sum_t w_t x_t B_t^T,
// where w_t is dt_t times the decay from t (exclusive) to the chunk end and
// T_c the chunk's decay, both 0 across a document boundary (page "State Space
// Duality and Mamba-2", "The SSD Block Decomposition Algorithm": the chunk
// states and their passing from chunk to chunk).  Each state is written to
// memory once and nothing else is, where a parallel pass over chunks plus a
// scan over them writes and reads every state again.  Per chunk the x and B
// rows are staged in LDS transposed to [row][token], so an MFMA operand (8
// consecutive tokens of a row, or 16 in fp32) is one or four 16-byte reads.
// bf16 inputs: w_t x_t as hi + lo bf16 (about 16 bits of the product) against
// the exact bf16 B rows, fp32 accumulation; fp32 inputs: fp32 MFMA.
constexpr int kStThreads = 256;

// MFMA results are read by vector code (the state stores, the decay) only
// after this: 7 wait states after a bf16 16x16x32 step, 12 after fp32 16x16x4.
// The empty statements place every accumulator's MFMAs before the wait (the
// volatile statements keep their order); the memory clobber keeps the state
// stores after it.
template <bool F32, int K>
__device__ inline void states_fence(f32x4 (&v)[K]) {
#pragma unroll
    for (int k = 1; k < K; ++k) asm volatile("" : "+v"(v[k]));
    if constexpr (F32)
        asm volatile("s_nop 7\n\ts_nop 3" : "+v"(v[0]) : : "memory");
    else
        asm volatile("s_nop 7" : "+v"(v[0]) : : "memory");
}

// One instantiation per (headdim, dstate): with the tile count known, the
// common shapes are straight-line code and the compiler's memory-wait counts
// stay exact (behind runtime-guarded tiles it waits for every store).  A
// state is stored right after its update, so the accumulators are next
// overwritten a whole chunk later: they are the stores' data registers, and
// rewriting them waits for those stores.
//
// Workgroups past batch * nheads walk the adjoint of a tail walk instead (see
// BwdArgs): G_{c-1} = T_c G_c + sum_t u_t dy_t C_t^T from dfinal over chunks
// nchunks - 1 down to split_chunk, u_t the decay from the chunk start through
// t (0 from a document boundary on, and past the end of the row), the form
// of the state walk with dy, C and u for x, B and w, in reverse.  Only the
// last G is stored, to g_tail.
template <typename IO, int P, int N>
__global__ __launch_bounds__(kStThreads, (P <= 32 || (P == 64 && std::is_same<IO, bf16>::value)) ? 3 : P == 64 ? 2 : 1)
void ssd_bwd_states_kernel(BwdArgs a, float *out) {
    constexpr int Q = kBwdQ, PBn = P / 16, NT = PBn * (N / 16);
    constexpr bool kBf = std::is_same<IO, bf16>::value;
    constexpr int MAXT = (NT + 3) / 4;                          // tiles per wave
    constexpr int TP = kBf ? Q + 8 : Q + 4;                     // row pitch: 144 or 272 bytes
    constexpr int EPV = 16 / (int)sizeof(IO);                   // elements per 16-byte piece
    constexpr int XP = Q * P / EPV, BP = Q * N / EPV;           // pieces per chunk
    constexpr int XPC = (XP + kStThreads - 1) / kStThreads, BPC = (BP + kStThreads - 1) / kStThreads;
    __shared__ __attribute__((aligned(16))) IO sX[kBf ? 2 : 1][P * TP];   // w x (bf16: hi, lo)
    __shared__ __attribute__((aligned(16))) IO sBt[N * TP];
    __shared__ float sw[Q];
    __shared__ float sT;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int H = a.nheads, L = a.seqlen, G = a.ngroups;
    const int nch = a.nchunks;
    const bool adj = (int)blockIdx.x >= a.batch * H;   // uniform: the workgroup's role
    const int tk = (int)blockIdx.x - a.batch * H;      // adjoint: tail walk tk
    const int bh = adj ? a.whole_units + tk : (int)blockIdx.x;
    const int b = bh / H, h = bh % H, grp = h / (H / G);
    constexpr int PN = P * N;
    const float A_h = a.A[h];
    const float *dt_row = a.dt + (int64_t)b * L * H + h;
    const int32_t *seq_row = a.seq_idx ? a.seq_idx + (int64_t)b * L : nullptr;
    float *outh = adj ? a.g_tail + (int64_t)tk * PN : out + (int64_t)bh * nch * PN;
    const IO *xg = (const IO *)(adj ? a.dy : a.x), *bg = (const IO *)(adj ? a.C : a.B);
    // the chunks walked: state 0 .. nch - 2 (every state stored), adjoint
    // nch - 1 down to split_chunk (the last G stored)
    const int nsteps = adj ? nch - a.split_chunk : nch - 1;
    auto chunk_of = [&](int s) { return adj ? nch - 1 - s : s; };

    // this wave's tiles: i = wave + 4 j, rows of p block i % PBn, columns of
    // n block i / PBn; lane holds rows 4 g + r, column l16
    auto valid = [&](int j) { return NT % 4 == 0 || wave + 4 * j < NT; };
    auto tile_off = [&](int j, int r) {
        const int i = wave + 4 * j;
        return ((i % PBn) * 16 + 4 * g + r) * N + (i / PBn) * 16 + l16;
    };
    f32x4 acc[MAXT];
    const float *h0 = adj ? (a.dfinal ? a.dfinal + (int64_t)bh * PN : nullptr)
                          : (a.init_states ? a.init_states + (int64_t)bh * PN : nullptr);
#pragma unroll
    for (int j = 0; j < MAXT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = (h0 && valid(j)) ? h0[tile_off(j, r)] : 0.f;
    auto store_state = [&](int c) {
        float *oc = outh + (int64_t)c * PN;
#pragma unroll
        for (int j = 0; j < MAXT; ++j)
            if (valid(j))
#pragma unroll
                for (int r = 0; r < 4; ++r) oc[tile_off(j, r)] = acc[j][r];
    };

    // chunk operands in 16-byte pieces, loaded a chunk ahead; rows past the
    // end of the row (only the adjoint walk stages the last chunk) are read
    // at the last valid token, and their weight is 0
    uint4 rx[XPC], rb[BPC];
    auto load_chunk = [&](int c) {
        const int64_t r0 = (int64_t)b * L + c * Q;
        const int tmax = min(Q, L - c * Q) - 1;
#pragma unroll
        for (int k = 0; k < XPC; ++k) {
            const int piece = tid + k * kStThreads;
            if (XP % kStThreads == 0 || piece < XP) {
                const int t = min(piece / (P / EPV), tmax), q = piece % (P / EPV);
                rx[k] = *(const uint4 *)(xg + ((r0 + t) * H + h) * P + q * EPV);
            }
        }
#pragma unroll
        for (int k = 0; k < BPC; ++k) {
            const int piece = tid + k * kStThreads;
            if (BP % kStThreads == 0 || piece < BP) {
                const int t = min(piece / (N / EPV), tmax), q = piece % (N / EPV);
                rb[k] = *(const uint4 *)(bg + ((r0 + t) * G + grp) * N + q * EPV);
            }
        }
    };
    // token values of a chunk (thread t < Q: token t), a chunk ahead; the
    // sequence indices are compared where the flag is used, so the loads need
    // not complete before the chunk's stores are issued
    float dtv = 0.f;
    int sq_cur = 0, sq_prev = 0;
    int tok_valid = 0;
    auto fetch_tokens = [&](int c) {
        const int t = c * Q + tid;
        tok_valid = t < L;
        dtv = 0.f;
        sq_cur = sq_prev = 0;
        if (tok_valid) {
            dtv = dt_row[(int64_t)t * H];
            if (seq_row) {
                sq_cur = seq_row[t];
                sq_prev = t > 0 ? seq_row[t - 1] : sq_cur;
            }
        }
    };
    if (nsteps > 0) {
        load_chunk(chunk_of(0));
        if (tid < Q) fetch_tokens(chunk_of(0));
    }
    if (!adj) store_state(0);
    for (int s = 0; s < nsteps; ++s) {
        const int c = chunk_of(s);
        // the token weights and T of chunk c: wave 0, lane = token, log2
        // decays summed over lanes.  State walk: w_t = dt_t 2^(sum after t),
        // 0 if a document starts after t.  Adjoint walk: u_t = 2^(sum through
        // t), 0 from a document start on.  T = 2^(sum), 0 if any starts.
        if (wave == 0) {
            const int flag = tok_valid && sq_cur != sq_prev;   // token t starts a document
            const float d = (flag || !tok_valid) ? 0.f : __fmul_rn(__fmul_rn(dtv, A_h), kLog2e);
            const unsigned long long m = __ballot(flag);
            float tot;
            if (!adj) {
                float sfx = d;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_down(sfx, off, 64);
                    if (lane + off < 64) sfx += o;
                }
                const float after = __shfl_down(sfx, 1, 64);   // sum over (t, 63]
                const bool cut = lane < 63 && (m >> (lane + 1)) != 0ull;
                sw[lane] = cut ? 0.f : dtv * __builtin_amdgcn_exp2f(lane < 63 ? after : 0.f);
                tot = sfx;                                     // lane 0: the whole sum
            } else {
                float pre = d;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(pre, off, 64);
                    if (lane >= off) pre += o;
                }
                const bool cut = (m & ((2ull << lane) - 1ull)) != 0ull;   // a start at or before t
                sw[lane] = (cut || !tok_valid) ? 0.f : __builtin_amdgcn_exp2f(pre);
                tot = __shfl(pre, 63, 64);                     // the whole sum
            }
            if (lane == 0) sT = m ? 0.f : __builtin_amdgcn_exp2f(tot);
        }
        __syncthreads();   // the last chunk's MFMAs are done with the tiles; w and T visible
        const float T = sT;
#pragma unroll
        for (int k = 0; k < XPC; ++k) {
            const int piece = tid + k * kStThreads;
            if (XP % kStThreads == 0 || piece < XP) {
                const int t = piece / (P / EPV), q0 = (piece % (P / EPV)) * EPV;
                const float wt = sw[t];
                if constexpr (kBf) {
                    const bf16x8 v8 = __builtin_bit_cast(bf16x8, rx[k]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = (float)v8[e] * wt;
                        const bf16 hi = (bf16)v;
                        sX[0][(q0 + e) * TP + t] = hi;
                        sX[1][(q0 + e) * TP + t] = (bf16)(v - (float)hi);
                    }
                } else {
                    const float4 v4 = __builtin_bit_cast(float4, rx[k]);
                    sX[0][(q0 + 0) * TP + t] = v4.x * wt;
                    sX[0][(q0 + 1) * TP + t] = v4.y * wt;
                    sX[0][(q0 + 2) * TP + t] = v4.z * wt;
                    sX[0][(q0 + 3) * TP + t] = v4.w * wt;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < BPC; ++k) {
            const int piece = tid + k * kStThreads;
            if (BP % kStThreads == 0 || piece < BP) {
                const int t = piece / (N / EPV), q0 = (piece % (N / EPV)) * EPV;
                if constexpr (kBf) {
                    const bf16x8 v8 = __builtin_bit_cast(bf16x8, rb[k]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) sBt[(q0 + e) * TP + t] = v8[e];
                } else {
                    const float4 v4 = __builtin_bit_cast(float4, rb[k]);
                    sBt[(q0 + 0) * TP + t] = v4.x;
                    sBt[(q0 + 1) * TP + t] = v4.y;
                    sBt[(q0 + 2) * TP + t] = v4.z;
                    sBt[(q0 + 3) * TP + t] = v4.w;
                }
            }
        }
        if (s + 1 < nsteps) {   // the next chunk is staged in the next pass
            load_chunk(chunk_of(s + 1));
            if (tid < Q) fetch_tokens(chunk_of(s + 1));
        }
        __syncthreads();   // staged tiles visible
#pragma unroll
        for (int j = 0; j < MAXT; ++j) {
            if (!valid(j)) continue;
            const int i = wave + 4 * j;
            const int prow = ((i % PBn) * 16 + l16) * TP, nrow = ((i / PBn) * 16 + l16) * TP;
            f32x4 v = acc[j] * T;
            if constexpr (kBf) {
#pragma unroll
                for (int ks = 0; ks < Q / 32; ++ks) {
                    const int k0 = 32 * ks + 8 * g;
                    const bf16x8 bb = *(const bf16x8 *)&sBt[nrow + k0];
                    v = mfma_bf16(*(const bf16x8 *)&sX[0][prow + k0], bb, v);
                    v = mfma_bf16(*(const bf16x8 *)&sX[1][prow + k0], bb, v);
                }
            } else {
                // step s, lane group g: token 16 g + s
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const float4 xa = *(const float4 *)&sX[0][prow + 16 * g + 4 * s4];
                    const float4 ba = *(const float4 *)&sBt[nrow + 16 * g + 4 * s4];
                    v = mfma_f32(xa.x, ba.x, v);
                    v = mfma_f32(xa.y, ba.y, v);
                    v = mfma_f32(xa.z, ba.z, v);
                    v = mfma_f32(xa.w, ba.w, v);
                }
            }
            acc[j] = v;
        }
        states_fence<!kBf>(acc);
        if (!adj) store_state(c + 1);
    }
    if (adj) store_state(0);   // g_tail[tk]: G at the end of chunk split_chunk - 1
}

void launch_bwd_states(bool bf16_io, const BwdArgs &a, float *out, hipStream_t stream) {
    const dim3 grid(a.batch * a.nheads + a.tail_units), block(kStThreads);
    auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, 0, stream, a, out); };
    auto by_n = [&](auto pc) {   // the API admits dstate 16, 32, 64 and 128
        constexpr int P = decltype(pc)::value;
        switch (a.dstate) {
        case 16: bf16_io ? go(ssd_bwd_states_kernel<bf16, P, 16>) : go(ssd_bwd_states_kernel<float, P, 16>); break;
        case 32: bf16_io ? go(ssd_bwd_states_kernel<bf16, P, 32>) : go(ssd_bwd_states_kernel<float, P, 32>); break;
        case 64: bf16_io ? go(ssd_bwd_states_kernel<bf16, P, 64>) : go(ssd_bwd_states_kernel<float, P, 64>); break;
        default: bf16_io ? go(ssd_bwd_states_kernel<bf16, P, 128>) : go(ssd_bwd_states_kernel<float, P, 128>); break;
        }
    };
    switch (a.headdim) {   // and headdim 16, 32, 64 and 128
    case 16: by_n(std::integral_constant<int, 16>{}); break;
    case 32: by_n(std::integral_constant<int, 32>{}); break;
    case 64: by_n(std::integral_constant<int, 64>{}); break;
    default: by_n(std::integral_constant<int, 128>{}); break;
    }
}

void launch_bwd(bool bf16_io, const BwdArgs &a, hipStream_t stream) {
    const dim3 grid(a.whole_units + 2 * a.tail_units), block(kBwdThreads);
    auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, 0, stream, a); };
    switch (a.headdim) {   // the API admits 16, 32, 64 and 128
    case 16: bf16_io ? go(ssd_bwd_kernel<bf16, 16>) : go(ssd_bwd_kernel<float, 16>); break;
    case 32: bf16_io ? go(ssd_bwd_kernel<bf16, 32>) : go(ssd_bwd_kernel<float, 32>); break;
    case 64: bf16_io ? go(ssd_bwd_kernel<bf16, 64>) : go(ssd_bwd_kernel<float, 64>); break;
    default: bf16_io ? go(ssd_bwd_kernel<bf16, 128>) : go(ssd_bwd_kernel<float, 128>); break;
    }
    const int64_t total = (int64_t)a.batch * a.seqlen * a.ngroups * a.dstate + a.nheads;
    hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, a);
}

}  // namespace ssd
