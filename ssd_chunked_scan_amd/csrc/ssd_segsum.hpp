// Hierarchy-aware segsum: the per-chunk decay factors of the SSD forward
// pass and the 1-semiseparable mask built from them.
//
// Page "GPU Hierarchy Meets Structured Matrices" (abstract) splits the
// chunk's decay mask L (page "State Space Duality and Mamba-2", "The
// Mathematical Bridge": L_ij = prod_{k=j+1..i} a_k for i >= j) into 1-SS
// diagonal blocks and rank-one off-diagonal blocks.  Here the sub-blocks are
// 16 tokens wide (the MFMA tile edge):
//
//   * log2-decays d_k = dt_k A_h log2(e) <= 0 are summed per sub-block with
//     nested sequential sums (every partial sum is the previous one plus a
//     term <= 0, so sums never increase and never cancel);
//   * a diagonal sub-block entry is 2^(direct sum over (j, i]) taken
//     leftwards from the diagonal;
//   * an off-diagonal entry of sub-block (I, J), J < I, is F(i, J) * W_j:
//     W_j = 2^(sum over (j, end of J]) is the sub-block suffix decay, and
//     F(i, J) = L at column (end of J), carried leftwards across sub-blocks by
//     F(i, J) = F(i, J+1) * Tb_{J+1}, Tb = whole-sub-block decay.  The chain
//     starts at F(i, I-1) = 2^(the row's direct sum extended over the first
//     token of block I).
//
// Every factor is 2^(sum of terms <= 0) in [0, 1] and every step multiplies
// by a factor in [0, 1] or adds a term <= 0, so along each row the mask is in
// [0, 1] and non-increasing away from the diagonal in fp32, for any input
// (Tb_{J+1} <= W at the first column of J+1 because Tb extends that column's
// nested suffix sum by one more non-positive term).
//
// Document boundaries (page "Parallel Scan and Hardware-Aware SSM Kernels",
// "When it breaks": mask a_k to zero at a boundary) enter by selecting a
// factor to exactly 0, never through -inf arithmetic.  The library is built
// with floating-point contraction off (hipcc otherwise fuses a * b + c into
// an FMA, even through __fmul_rn / __fadd_rn), so every term is rounded
// before it is added and every kernel that includes this header produces
// bit-identical factors and mask values.
#pragma once

#include "ssd_common.hpp"

namespace ssd {

// Per-chunk segsum values in LDS.  Q = chunk size (multiple of 16, <= 256).
template <int Q>
struct SegLds {
    static constexpr int NB = Q / 16;
    float d[Q];      // log2-decay of token t (0 past the end of the row)
    float dt[Q];     // dt of token t (0 past the end)
    float W[Q];      // sub-block suffix decay over (t, end of t's sub-block]
    float u[Q];      // decay from the previous chunk's state to token t: prod_{k<=t} a_k
    float wcd[Q];    // decay from token t to the chunk end, times dt_t
    int rs[Q];       // last reset position <= t in the chunk, -1 if none
    int flag[Q];     // 1 if the state resets at token t (document boundary)
    float Tb[NB];    // whole-sub-block decay (0 if a reset lies inside)
    int blast[NB];   // last reset position inside sub-block, -1 if none
    float T;         // whole-chunk decay (0 if a reset lies inside)
    int any_reset;   // 1 if some token of the chunk resets the state
};

// Step 1a, thread t < Q: read token t's dt and reset flag from global memory
// (dt = 0 and no reset past the end of the row).  t0 = chunk start, nvalid =
// tokens of the chunk inside the row.  A reset happens at global token t > 0
// where seq_idx changes.
__device__ inline void seg_fetch_token(int t, int t0, int nvalid, const float *dt_row,
                                       int dt_stride, const int32_t *seq_row, float &dtv,
                                       int &flag) {
    dtv = 0.f;
    flag = 0;
    if (t < nvalid) {
        dtv = dt_row[(int64_t)(t0 + t) * dt_stride];
        if (seq_row && (t0 + t) > 0) flag = seq_row[t0 + t] != seq_row[t0 + t - 1];
    }
}

// Step 1b, thread t < Q: token values in LDS.
template <int Q>
__device__ inline void seg_store_token(SegLds<Q> &s, int t, float dtv, float A_h, int flag) {
    s.d[t] = __fmul_rn(__fmul_rn(dtv, A_h), kLog2e);
    s.dt[t] = dtv;
    s.flag[t] = flag;
}

// Step 1 in one go (fetch + store), for kernels that do not prefetch.
template <int Q>
__device__ inline void seg_load_token(SegLds<Q> &s, int t, int t0, int nvalid,
                                      const float *dt_row, int dt_stride,
                                      float A_h, const int32_t *seq_row, const DtMap &dm) {
    float dtv;
    int flag;
    seg_fetch_token(t, t0, nvalid, dt_row, dt_stride, seq_row, dtv, flag);
    if (t < nvalid) dtv = dt_apply(dm, dtv);
    seg_store_token<Q>(s, t, dtv, A_h, flag);
}

// Step 2, thread t < Q (after a barrier): nested sums inside t's sub-block.
template <int Q>
__device__ inline void seg_block_sums(SegLds<Q> &s, int t) {
    const int B0 = t & ~15;
    float pre = 0.f;
    int lastin = -1;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
        const int k = B0 + kk;
        if (k <= t) {
            pre = __fadd_rn(pre, s.d[k]);
            if (s.flag[k]) lastin = k;
        }
    }
    float suf = 0.f;
    int fsuf = 0;
#pragma unroll
    for (int kk = 15; kk >= 1; --kk) {
        const int k = B0 + kk;
        if (k > t) {
            suf = __fadd_rn(suf, s.d[k]);
            fsuf |= s.flag[k];
        }
    }
    // Decay of the prefix [B0, t]; stored in u[] and finished in step 3.
    s.u[t] = (lastin >= 0) ? 0.f : __builtin_amdgcn_exp2f(pre);
    s.W[t] = fsuf ? 0.f : __builtin_amdgcn_exp2f(suf);
    s.rs[t] = lastin;
    if (t == B0) {
        const float tau = __fadd_rn(suf, s.d[B0]);
        s.Tb[t >> 4] = (fsuf | s.flag[B0]) ? 0.f : __builtin_amdgcn_exp2f(tau);
    }
    if (t == B0 + 15) s.blast[t >> 4] = lastin;
}

// Step 3, thread t < Q (after a barrier): cross-sub-block products.
template <int Q>
__device__ inline void seg_chunk_products(SegLds<Q> &s, int t) {
    constexpr int NB = Q / 16;
    const int K = t >> 4;
    float V = 1.f;
    for (int k = 0; k < K; ++k) V = __fmul_rn(V, s.Tb[k]);
    float Z = 1.f;
    for (int k = NB - 1; k > K; --k) Z = __fmul_rn(Z, s.Tb[k]);
    s.u[t] = __fmul_rn(s.u[t], V);
    s.wcd[t] = __fmul_rn(__fmul_rn(s.W[t], Z), s.dt[t]);
    if (s.any_reset) {
        int rs = s.rs[t];
        if (rs < 0)
            for (int k = 0; k < K; ++k)
                if (s.blast[k] >= 0) rs = s.blast[k];
        s.rs[t] = rs;
    }
    if (t == 0) {
        float T = 1.f;
        for (int k = 0; k < NB; ++k) T = __fmul_rn(T, s.Tb[k]);
        s.T = T;
    }
}

// ---------------------------------------------------------------------------
// Wave form of steps 1-2 for the bf16 kernels: thread t < Q owns token t, and
// a 16-lane DPP row of its wave is one sub-block.  The nested sums are built
// by repeated row shifts (DPP row_shl:1 hands each lane the value of the next
// lane of its row, 0 past the row end): after k rounds of e <- shl1(e) + d,
// lane t holds the nested sum from the end of the sub-block down to t over up
// to k + 1 terms, accumulated in exactly the order of the sequential loop of
// seg_block_sums, so W and Tb are bit-identical to it.

// Per-chunk segsum values of the bf16 kernels in LDS.
template <int Q>
struct SegBuf {
    static constexpr int NB = Q / 16;
    float d[Q];       // log2-decay of token t (0 past the end of the row)
    float dt[Q];      // dt of token t (0 past the end)
    float wd[Q];      // W_t * dt_t: decay to the end of t's sub-block, times dt
    int last1[Q];     // 1 + last reset position <= t inside t's sub-block, 0 if none
    float Tb[NB];     // whole-sub-block decay (0 if a reset lies inside)
    int blast1[NB];   // 1 + last reset position inside the sub-block, 0 if none
    float Tp[NB / 2]; // decay over 32-token pair m: Tb[2m] * Tb[2m+1]
};

// Debug record of one chunk's segsum factors (32-bit words): the values the
// bf16 head kernel keeps in SegBuf, in a layout both segsum paths can write,
// so that the DPP sums of seg_tokens can be compared bit for bit with the
// sequential sums of seg_block_sums.  last1 and blast1 are int32 words.
template <int Q>
struct SegRecord {
    static constexpr int NB = Q / 16;
    static constexpr int D = 0, DT = Q, WD = 2 * Q, LAST1 = 3 * Q, TB = 4 * Q, BLAST1 = 4 * Q + NB,
                         TP = 4 * Q + 2 * NB, WORDS = 4 * Q + 2 * NB + NB / 2;
};

template <int CTRL>
__device__ inline int dpp_row(int v) {
    // row_mask and bank_mask 0xf; lanes whose source lies outside the row read 0
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}
constexpr int kDppRowShl1 = 0x101;
constexpr int kDppRowShr1 = 0x111;

__device__ inline float dpp_row_shl1(float v) {
    return __builtin_bit_cast(float, dpp_row<kDppRowShl1>(__builtin_bit_cast(int, v)));
}

// Steps 1-2 for token t (thread t < Q; whole waves only): dtv and flag are
// the token's dt and reset flag (0 past the end of the row).  resets is
// uniform: false when the call has no seq_idx.
// rec (nullable): the chunk's SegRecord in global memory, written as well.
template <int Q>
__device__ inline void seg_tokens(SegBuf<Q> &s, int t, float dtv, int flag, float A_h,
                                  bool resets, float *rec = nullptr) {
    const float d = __fmul_rn(__fmul_rn(dtv, A_h), kLog2e);
    float e = d;
#pragma unroll
    for (int k = 0; k < 15; ++k) e = __fadd_rn(dpp_row_shl1(e), d);
    // e = sum over [t, end of sub-block]; the suffix (t, end] is the next lane's e
    const float suf = dpp_row_shl1(e);
    int fsuf = 0, last1 = 0;
    if (resets) {
        // 1 + last reset position <= t in the sub-block: running max to the right
        int v = flag ? t + 1 : 0;
        v = max(v, dpp_row<kDppRowShr1>(v));
        v = max(v, dpp_row<kDppRowShr1 + 1>(v));
        v = max(v, dpp_row<kDppRowShr1 + 3>(v));
        v = max(v, dpp_row<kDppRowShr1 + 7>(v));
        last1 = v;
        // any reset in (t, end of sub-block]: running OR to the left of the
        // next lanes' flags
        int f = dpp_row<kDppRowShl1>(flag);
        f |= dpp_row<kDppRowShl1>(f);
        f |= dpp_row<kDppRowShl1 + 1>(f);
        f |= dpp_row<kDppRowShl1 + 3>(f);
        f |= dpp_row<kDppRowShl1 + 7>(f);
        fsuf = f;
        s.last1[t] = last1;
        if ((t & 15) == 15) s.blast1[t >> 4] = last1;
    }
    const float W = fsuf ? 0.f : __builtin_amdgcn_exp2f(suf);
    s.d[t] = d;
    s.dt[t] = dtv;
    s.wd[t] = __fmul_rn(W, dtv);
    // meaningful on the first lane of each sub-block
    const float tb = (fsuf | flag) ? 0.f : __builtin_amdgcn_exp2f(e);
    if ((t & 15) == 0) s.Tb[t >> 4] = tb;
    // the first lane of each 32-token pair takes the decay of the pair's
    // second sub-block from 16 lanes up (same wave: waves own 64 tokens)
    const float tb_hi = __shfl_down(tb, 16, 64);
    const float tp = __fmul_rn(tb, tb_hi);
    if ((t & 31) == 0) s.Tp[t >> 5] = tp;
    if (rec) {
        using R = SegRecord<Q>;
        rec[R::D + t] = d;
        rec[R::DT + t] = dtv;
        rec[R::WD + t] = __fmul_rn(W, dtv);
        rec[R::LAST1 + t] = __builtin_bit_cast(float, last1);
        if ((t & 15) == 0) rec[R::TB + (t >> 4)] = tb;
        if ((t & 15) == 15) rec[R::BLAST1 + (t >> 4)] = __builtin_bit_cast(float, last1);
        if ((t & 31) == 0) rec[R::TP + (t >> 5)] = tp;
    }
}

// Step 3 in registers (every wave after a barrier): the cross-sub-block
// prefix products V_I = Tb_0 ... Tb_{I-1} for the row tiles I = Irow[k] and
// the chunk decay T, multiplied in the order of seg_chunk_products (the
// suffix products are formed on the fly by the callers, also in that order).
template <int NB, int K>
__device__ inline void seg_prefix_products(const float (&Tb)[NB], const int (&Irow)[K],
                                           float (&VI)[K], float &T) {
    float V = 1.f;
#pragma unroll
    for (int k = 0; k < K; ++k) VI[k] = 1.f;
#pragma unroll
    for (int j = 1; j <= NB; ++j) {
        V = __fmul_rn(V, Tb[j - 1]);
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (j < NB && Irow[k] == j) VI[k] = V;
    }
    T = V;
}

// Last reset position <= i in the chunk (-1 if none); I = i / 16.
template <int Q>
__device__ inline int seg_last_reset(const SegBuf<Q> &s, int i, int I) {
    int r = s.last1[i];
    if (r == 0)
        for (int k = 0; k < I; ++k) r = max(r, s.blast1[k]);
    return r - 1;
}

// Diagonal sub-block of row i (sub-block start I0), in the MFMA accumulator
// layout: the lane holds columns j = I0 + 4g + r, r = 0..3.  e[r] receives the
// direct sum over (j, i] (meaningful for j <= i); the return value is the sum
// over [I0, i], the start of the off-diagonal chain.
__device__ inline float seg_diag_row(const float *d, int I0, int i, int g, float e[4]) {
    float acc = 0.f;
#pragma unroll
    for (int kk = 15; kk >= 0; --kk) {
        if ((kk >> 2) == g) e[kk & 3] = acc;
        const float dk = d[I0 + kk];
        acc = (I0 + kk <= i) ? __fadd_rn(acc, dk) : acc;
    }
    return acc;
}

// seg_diag_row with the sub-block's log2-decays already in registers
// (dd[kk] = d[I0 + kk]); the same additions in the same order.
__device__ inline float seg_diag_row_regs(const float (&dd)[16], int I0, int i, int g, float e[4]) {
    float acc = 0.f;
#pragma unroll
    for (int kk = 15; kk >= 0; --kk) {
        if ((kk >> 2) == g) e[kk & 3] = acc;
        acc = (I0 + kk <= i) ? __fadd_rn(acc, dd[kk]) : acc;
    }
    return acc;
}

// Mask value of a diagonal-sub-block entry (i, j) from its direct sum.
__device__ inline float seg_diag_value(float e, int i, int j, int rs_i) {
    return (j > i || rs_i > j) ? 0.f : __builtin_amdgcn_exp2f(e);
}

// Start of the off-diagonal chain for row i: F(i, I-1) = prod_{k=I0..i} a_k.
__device__ inline float seg_chain_start(float sum_I0_i, int I0, int rs_i) {
    return (rs_i >= I0) ? 0.f : __builtin_amdgcn_exp2f(sum_I0_i);
}

// F(i, J) from F(i, J+1) and the decay of sub-block J+1.
__device__ inline float seg_chain_step(float F, float Tb_next) { return __fmul_rn(F, Tb_next); }

// Off-diagonal mask entry L_ij = F(i, J) * W_j.
__device__ inline float seg_offdiag(float F, float W) { return __fmul_rn(F, W); }

}  // namespace ssd
