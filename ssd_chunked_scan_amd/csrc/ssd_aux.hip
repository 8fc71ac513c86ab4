// Auxiliary kernels of the SSD forward pass:
//  * the inter-split state scan that joins sequence-parallel splits, and
//  * the debug export of the decay mask exactly as the chunk kernels build it.
#include "ssd_common.hpp"
#include "ssd_segsum.hpp"

namespace ssd {

// Entering state of every split.  Split s holds its local end state (from a
// zero state) and its decay T_s; the affine composition of page "Parallel
// Scan and Hardware-Aware SSM Kernels" ("The scan": applying (A1, b1) then
// (A2, b2) gives (A2 A1, A2 b1 + b2)) walked sequentially over the splits of
// one row gives E_0 = init, E_{s+1} = T_s E_s + local_s.  Each slot is
// overwritten by the entering state of its split.  One thread per state
// element; the split count is small, so the walk is short.
__global__ __launch_bounds__(256) void ssd_split_scan_kernel(const float *init_states,
                                                              float *ws_states,
                                                              const float *ws_decay,
                                                              int batch, int nheads, int nsplits,
                                                              int pn) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)batch * nheads * pn;
    if (e >= total) return;
    const int64_t bh = e / pn, k = e % pn;
    float E = init_states ? init_states[bh * pn + k] : 0.f;
    // Groups of splits: all loads of a group are issued before its stores
    // (a store to ws_states could otherwise alias the next load, and each
    // split would wait a full memory round trip).
    constexpr int GRP = 16;   // the planner's split counts fit one group
    for (int s0 = 0; s0 < nsplits; s0 += GRP) {
        float loc[GRP], T[GRP];
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            const int s = s0 + u;
            loc[u] = 0.f;
            T[u] = 0.f;
            if (s + 1 < nsplits) {
                loc[u] = ws_states[(bh * nsplits + s) * pn + k];
                T[u] = ws_decay[bh * nsplits + s];
            }
        }
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            const int s = s0 + u;
            if (s < nsplits) {
                ws_states[(bh * nsplits + s) * pn + k] = E;
                if (s + 1 < nsplits) E = fmaf(T[u], E, loc[u]);
            }
        }
    }
}

void launch_split_scan(const float *init_states, float *ws_states, const float *ws_decay,
                       int batch, int nheads, int nsplits, int pn, hipStream_t stream) {
    const int64_t total = (int64_t)batch * nheads * pn;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    hipLaunchKernelGGL(ssd_split_scan_kernel, grid, block, 0, stream, init_states, ws_states,
                       ws_decay, batch, nheads, nsplits, pn);
}

// One workgroup per (batch row * head, chunk).  VARIANT selects how the mask
// entries L_ij = 2^(sum of d_k over (j, i]) are evaluated (page "GPU Hierarchy
// Meets Structured Matrices", abstract, names the three):
//   kSegsumHierarchy  the forward kernels' construction: nested sums inside
//                     16-token sub-blocks, rank-one factors across them (same
//                     steps and per-lane order as the bf16 chunk kernel: each
//                     wave takes 16-row tiles, each lane one row i and columns
//                     16 jt + 4 g + r, the F chain walked leftwards);
//   kSegsumDirect     the dense "direct segsum": thread j owns column j and
//                     keeps the running sum over (j, i] as i grows, one exp per
//                     entry (Q^2/2 of them);
//   kSegsumDiff       the "diff segsum": inclusive prefix sums cs over the
//                     chunk by an associative scan, entry 2^(cs_i - cs_j)
//                     (prefix subtraction).
// Document boundaries zero an entry by select in all three.  With out ==
// nullptr only the per-chunk sums are written (the evaluation without the
// mask's HBM traffic, for timing).
template <int Q, int VARIANT>
__global__ __launch_bounds__(kThreads) void ssd_mask_kernel(MaskArgs m) {
    constexpr int NB = Q / 16;
    __shared__ __attribute__((aligned(16))) SegLds<Q> sg;
    __shared__ float cs[Q];
    __shared__ float block_sum;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x;
    const int b = bh / m.nheads, h = bh % m.nheads;
    const int ci = blockIdx.y;
    const int c = m.chunk_begin + ci;
    const int L = m.seqlen, H = m.nheads;
    const int t0 = c * Q;
    const int nvalid = max(0, min(Q, L - t0));
    const float *dt_row = m.dt + (int64_t)b * L * H + h;
    const int32_t *seq_row = m.seq_idx ? m.seq_idx + (int64_t)b * L : nullptr;

    int flag_any = 0;
    if (tid < Q) {
        seg_load_token<Q>(sg, tid, t0, nvalid, dt_row, H, m.A[h], seq_row, dt_map_identity());
        flag_any = sg.flag[tid];
    }
    flag_any = __syncthreads_or(flag_any);
    if (tid == 0) sg.any_reset = flag_any;
    if (tid < Q) seg_block_sums<Q>(sg, tid);
    __syncthreads();
    if (m.factors && tid < Q) {
        // the block-sum path's factors in the head kernel's terms (before
        // seg_chunk_products turns rs into chunk-wide reset positions)
        using R = SegRecord<Q>;
        float *rec = m.factors + (((int64_t)b * H + h) * m.count + ci) * R::WORDS;
        const int t = tid;
        rec[R::D + t] = sg.d[t];
        rec[R::DT + t] = sg.dt[t];
        rec[R::WD + t] = __fmul_rn(sg.W[t], sg.dt[t]);
        rec[R::LAST1 + t] = __builtin_bit_cast(float, sg.rs[t] + 1);
        if ((t & 15) == 0) rec[R::TB + (t >> 4)] = sg.Tb[t >> 4];
        if ((t & 15) == 15) rec[R::BLAST1 + (t >> 4)] = __builtin_bit_cast(float, sg.blast[t >> 4] + 1);
        if ((t & 31) == 0) rec[R::TP + (t >> 5)] = __fmul_rn(sg.Tb[t >> 4], sg.Tb[(t >> 4) + 1]);
    }
    if (tid < Q) seg_chunk_products<Q>(sg, tid);
    __syncthreads();

    if (!m.out && !m.sums) return;   // factors only
    if (tid == 0) block_sum = 0.f;
    float *out = m.out ? m.out + (((int64_t)b * H + h) * m.count + ci) * Q * Q : nullptr;
    float csum = 0.f;
    if constexpr (VARIANT == kSegsumDirect || VARIANT == kSegsumDiff) {
        if constexpr (VARIANT == kSegsumDiff) {
            // inclusive prefix sums by an associative (Kogge-Stone) scan, as
            // chunkwise kernels compute them: each token's sum is grouped
            // differently, so the sums need not be monotone in fp32
            if (tid < Q) cs[tid] = sg.d[tid];
            __syncthreads();
            for (int off = 1; off < Q; off *= 2) {
                const float v = (tid < Q && tid >= off) ? cs[tid - off] : 0.f;
                __syncthreads();
                if (tid < Q && tid >= off) cs[tid] = __fadd_rn(cs[tid], v);
                __syncthreads();
            }
        }
        // thread j: column j, rows i = 0 .. Q-1 (a row is written by
        // consecutive threads)
        const int j = tid;
        if (j < Q) {
            float run = 0.f;
            bool cut = false;
            for (int i = 0; i < Q; ++i) {
                float v = 0.f;
                if (i >= j) {
                    if (VARIANT == kSegsumDirect && i > j) {
                        run = __fadd_rn(run, sg.d[i]);
                        cut = cut || sg.flag[i];
                        v = cut ? 0.f : __builtin_amdgcn_exp2f(run);
                    } else if (VARIANT == kSegsumDirect) {
                        v = 1.f;
                    } else {
                        v = (sg.rs[i] > j) ? 0.f : __builtin_amdgcn_exp2f(__fsub_rn(cs[i], cs[j]));
                    }
                }
                if (i >= nvalid || j >= nvalid) v = 0.f;
                csum += v;
                if (out) out[(int64_t)i * Q + j] = v;
            }
        }
    } else
    for (int I = wave; I < NB; I += 4) {
        const int i = I * 16 + l16;
        const int rs_i = sg.rs[i];
        float e[4];
        const float sum0 = seg_diag_row(sg.d, I * 16, i, g, e);
        float F = seg_chain_start(sum0, I * 16, rs_i);
        for (int jt = NB - 1; jt >= 0; --jt) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (jt == I) {
                for (int r = 0; r < 4; ++r) v[r] = seg_diag_value(e[r], i, jt * 16 + 4 * g + r, rs_i);
            } else if (jt < I) {
                if (jt < I - 1) F = seg_chain_step(F, sg.Tb[jt + 1]);
                for (int r = 0; r < 4; ++r) v[r] = seg_offdiag(F, sg.W[jt * 16 + 4 * g + r]);
            }
            for (int r = 0; r < 4; ++r)
                if (i >= nvalid || jt * 16 + 4 * g + r >= nvalid) v[r] = 0.f;
            csum += (v[0] + v[1]) + (v[2] + v[3]);
            // element (i, j): row i, columns j = 16 jt + 4 g .. +3
            if (out) *(f32x4 *)(out + (int64_t)i * Q + jt * 16 + 4 * g) = v;
        }
    }
    if (m.sums) {
        __syncthreads();
        atomicAdd(&block_sum, csum);
        __syncthreads();
        if (tid == 0) m.sums[((int64_t)b * H + h) * m.count + ci] = block_sum;
    }
}

template <int Q>
static void launch_mask_q(const MaskArgs &m, hipStream_t stream) {
    const dim3 grid(m.batch * m.nheads, m.count), block(kThreads);
    switch (m.variant) {
    case kSegsumDirect: hipLaunchKernelGGL((ssd_mask_kernel<Q, kSegsumDirect>), grid, block, 0, stream, m); break;
    case kSegsumDiff: hipLaunchKernelGGL((ssd_mask_kernel<Q, kSegsumDiff>), grid, block, 0, stream, m); break;
    default: hipLaunchKernelGGL((ssd_mask_kernel<Q, kSegsumHierarchy>), grid, block, 0, stream, m); break;
    }
}

void launch_mask(int Q, const MaskArgs &m, hipStream_t stream) {
    switch (Q) {
    case 64: launch_mask_q<64>(m, stream); break;
    case 128: launch_mask_q<128>(m, stream); break;
    default: launch_mask_q<256>(m, stream); break;
    }
}

}  // namespace ssd

namespace ssd {

// Exhaustive check of the hardware exp2 (v_exp_f32, the only exponential the
// decay factors use) over a range of fp32 bit patterns.  The mask stays in
// [0, 1] and non-increasing along rows only if exp2 is monotone and <= 1 on
// non-positive inputs (page "GPU Hierarchy Meets Structured Matrices",
// abstract: segsum without monotonicity violations).  Thread t takes the
// patterns [first + t span, first + (t+1) span) of the range [first, first +
// count), plus the pattern before its first one, and counts, for patterns
// u and u + 1 in its part: exp2(f(u+1)) > exp2(f(u)) when f(u+1) < f(u)
// (negative floats: a larger pattern is a smaller value), values above 1,
// values below 0 or NaN.  Plain vector stores of one counter triple per
// thread; the host sums them.
__global__ __launch_bounds__(256) void ssd_exp2_probe_kernel(uint32_t first, uint32_t count,
                                                             uint32_t span, uint32_t *out,
                                                             uint32_t nthreads) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= nthreads) return;
    const uint64_t lo = (uint64_t)t * span;
    const uint64_t hi = lo + span < (uint64_t)count ? lo + span : (uint64_t)count;
    uint32_t up = 0, above = 0, bad = 0;
    if (lo < hi) {
        float prev = __builtin_amdgcn_exp2f(__builtin_bit_cast(float, first + (uint32_t)(lo > 0 ? lo - 1 : 0)));
        for (uint64_t k = lo; k < hi; ++k) {
            const float x = __builtin_bit_cast(float, first + (uint32_t)k);
            const float v = __builtin_amdgcn_exp2f(x);
            // within the negative range a larger bit pattern is a smaller x
            if (k > 0 && v > prev) ++up;
            if (v > 1.f) ++above;
            if (!(v >= 0.f)) ++bad;
            prev = v;
        }
    }
    out[3 * (uint64_t)t + 0] = up;
    out[3 * (uint64_t)t + 1] = above;
    out[3 * (uint64_t)t + 2] = bad;
}

void launch_exp2_probe(uint32_t first, uint32_t count, uint32_t span, uint32_t *out, uint32_t nthreads,
                       hipStream_t stream) {
    hipLaunchKernelGGL(ssd_exp2_probe_kernel, dim3((nthreads + 255) / 256), dim3(256), 0, stream, first,
                       count, span, out, nthreads);
}

}  // namespace ssd
