// Single-token decode step: the SSM recurrence of page "State Space Duality
// and Mamba-2" ("The Mathematical Bridge"), one token, per head h:
//
//   a = exp(dt A_h)          h <- a h + dt x B^T          y = h C + D_h x
//
// (dt through the fused map and y through the silu(z) gate when they are
// enabled, as in the forward pass) with the N x P state carried in fp32 between calls (the final_states of the
// forward pass are its input).  The step is memory-bound: the state is read
// and written once (2 * 4 P N bytes per head), everything else is a few
// hundred bytes.  One workgroup per (batch row, head); the state is walked as
// rows of N/4 float4 (one row per N/4 lanes), the row sum of h C reduced
// across those lanes.
#include "ssd_common.hpp"

namespace ssd {

template <typename IO>
__device__ inline float io_load(const IO *p, int64_t i);
template <>
__device__ inline float io_load<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ inline float io_load<bf16>(const bf16 *p, int64_t i) { return (float)p[i]; }

template <typename IO>
__device__ inline void io_store(IO *p, int64_t i, float v);
template <>
__device__ inline void io_store<float>(float *p, int64_t i, float v) { p[i] = v; }
template <>
__device__ inline void io_store<bf16>(bf16 *p, int64_t i, float v) { p[i] = (bf16)v; }

template <typename IO, int N>
__global__ __launch_bounds__(256) void ssd_decode_kernel(DecodeArgs a) {
    constexpr int LPR = N / 4;          // lanes per state row (float4 each)
    constexpr int RPP = 256 / LPR;      // rows per pass of the workgroup
    const int bh = blockIdx.x;
    const int b = bh / a.nheads, h = bh % a.nheads;
    const int grp = h / (a.nheads / a.ngroups);
    const int P = a.headdim;
    const int tid = threadIdx.x, n4 = tid % LPR, r0 = tid / LPR;

    const float dt = dt_apply(dt_map_of(a, h), a.dt[bh]);
    const IO *zrow = (const IO *)a.z + (int64_t)bh * P;   // used only when a.z is set
    // the same per-token decay as the forward kernels: 2^(dt A log2 e)
    const float decay = __builtin_amdgcn_exp2f(__fmul_rn(__fmul_rn(dt, a.A[h]), kLog2e));
    const float Dh = a.D ? a.D[h] : 0.f;
    const IO *xrow = (const IO *)a.x + (int64_t)bh * P;
    const IO *Brow = (const IO *)a.B + ((int64_t)b * a.ngroups + grp) * N;
    const IO *Crow = (const IO *)a.C + ((int64_t)b * a.ngroups + grp) * N;
    f32x4 Bv, Cv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        Bv[r] = io_load(Brow, 4 * n4 + r);
        Cv[r] = io_load(Crow, 4 * n4 + r);
    }
    f32x4 *st = (f32x4 *)(a.state + (int64_t)bh * P * N);
    for (int p = r0; p < P; p += RPP) {
        const float xp = io_load(xrow, p);
        const float dx = dt * xp;
        f32x4 hv = st[(int64_t)p * LPR + n4];
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hv[r] = fmaf(decay, hv[r], dx * Bv[r]);
            part = fmaf(hv[r], Cv[r], part);
        }
        st[(int64_t)p * LPR + n4] = hv;
        // row sum over the LPR lanes of this row (aligned groups of LPR lanes)
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, LPR);
        if (n4 == 0) {
            float out = fmaf(Dh, xp, part);
            if (a.z) out *= silu_f32(io_load(zrow, p));   // fused output gate
            io_store((IO *)a.y, (int64_t)bh * P + p, out);
        }
    }
}

#define SSD_DECODE_CASE(T, n)                                                                  \
    if (N == n) {                                                                               \
        hipLaunchKernelGGL((ssd_decode_kernel<T, n>), dim3(a.batch * a.nheads), dim3(256), 0,  \
                           stream, a);                                                          \
        return true;                                                                            \
    }

bool launch_decode(bool bf16_io, int N, const DecodeArgs &a, hipStream_t stream) {
    if (bf16_io) {
        SSD_DECODE_CASE(bf16, 16) SSD_DECODE_CASE(bf16, 32) SSD_DECODE_CASE(bf16, 64) SSD_DECODE_CASE(bf16, 128)
    } else {
        SSD_DECODE_CASE(float, 16) SSD_DECODE_CASE(float, 32) SSD_DECODE_CASE(float, 64) SSD_DECODE_CASE(float, 128)
    }
    return false;
}

}  // namespace ssd
