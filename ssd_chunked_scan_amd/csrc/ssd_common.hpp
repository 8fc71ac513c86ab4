// Shared definitions of the gfx950 SSD forward kernels: argument block,
// vector types, bf16 helpers and the workgroup -> work-unit map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;  // four wave64s per workgroup

enum Mode : int {
    kModeFull = 0,        // outputs y; carries the state; last split writes final_states
    kModeSplitLocal = 1   // only the split's local end state and decay (zero entry state)
};

// Argument block shared by the chunk kernels (passed by value).
struct ChunkArgs {
    const void *x;
    const float *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;            // nullable
    const int32_t *seq_idx;    // nullable
    const float *init_states;  // nullable
    void *y;
    float *final_states;       // nullable
    float *ws_states;          // [batch][nheads][nsplits][headdim][dstate]
    float *ws_decay;           // [batch][nheads][nsplits]
    const void *ws_S;          // per-group C B^T blocks (bf16 path)
    const void *ws_BT;         // per-group token-transposed B (bf16 path)
    const void *ws_C;          // per-group C in operand order (bf16 path)
    int batch, seqlen, nheads, headdim, dstate, ngroups;
    int chunk;                 // chunk_size Q
    int nchunks;               // ceil(seqlen / Q)
    int nsplits;               // sequence-parallel splits per row
    int split_chunks;          // chunks per split
    int npblocks;              // headdim blocks per head
    int pblock;                // headdim columns per block
    int mode;                  // Mode
    int units;                 // batch * nheads * nsplits * npblocks
    int half_units;            // the last half_units units run as two workgroups,
                               // one per half of the headdim block (grid = units + half_units)
    // Fused prologue and epilogue (off when zero / null).
    const float *dt_bias;      // [nheads], nullable: dt <- dt + dt_bias[h]
    const void *z;             // [batch][seqlen][nheads][headdim] io dtype, nullable: y <- y silu(z)
    int dt_softplus;           // nonzero: dt <- softplus(dt)
    int dt_clamp;              // nonzero: dt <- min(max(dt, dt_lo), dt_hi)
    float dt_lo, dt_hi;
    int segsum_variant;        // SegsumVariant of the intra-chunk mask (fp32 kernel; bf16
                               // full pass at chunk 256)
    float *dbg_seg;            // nullable: the bf16 head kernel writes each chunk's segsum
                               // factors here (SegRecord layout, [batch][nheads][nchunks])
};

// Map from a raw per-token value to the step size dt of one head: plus the
// head's bias, then softplus, then the clamp, each step only when enabled.
// With no bias, no softplus and no clamp it returns the value unchanged.
struct DtMap {
    float bias;
    int softplus, clamp;
    float lo, hi;
};

template <typename Args>
__device__ inline DtMap dt_map_of(const Args &a, int h) {
    DtMap m;
    m.bias = a.dt_bias ? a.dt_bias[h] : 0.f;
    m.softplus = a.dt_softplus;
    m.clamp = a.dt_clamp;
    m.lo = a.dt_lo;
    m.hi = a.dt_hi;
    return m;
}

__device__ inline DtMap dt_map_identity() { return DtMap{0.f, 0, 0, 0.f, 0.f}; }

// softplus(v) = log(1 + e^v); above v = 20 it equals v to within e^-20 / v
// (below fp32 resolution), which also keeps e^v finite.
__device__ inline float softplus_f32(float v) { return v > 20.f ? v : log1pf(expf(v)); }

__device__ inline float dt_apply(const DtMap &m, float raw) {
    float v = m.bias != 0.f ? __fadd_rn(raw, m.bias) : raw;
    if (m.softplus) v = softplus_f32(v);
    if (m.clamp) v = fminf(fmaxf(v, m.lo), m.hi);
    return v;
}

// silu(z) = z / (1 + e^-z); for very negative z the reciprocal goes to 0
// and so does the product.
__device__ inline float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// Arguments of the per-group operand kernel (bf16 path).
struct CbArgs {
    const void *B;
    const void *C;
    void *ws_S;    // [batch][ngroups][nchunks][CbShape<Q>::NBLK][64 lanes] x 16 bytes
    void *ws_BT;   // [batch][ngroups][nchunks][Q/32][dstate][4] x 16 bytes
    void *ws_C;    // [batch][ngroups][nchunks][Q/16][KN][64 lanes] x 16 bytes,
                   // KN = max(dstate, 32) / 32
    int batch, seqlen, ngroups, nchunks;
};

// Layout of the per-group C B^T blocks of one chunk: for each 16-token row
// tile I, the blocks of its 32-token column pairs m = 0 .. I/2.
template <int Q>
struct CbShape {
    static constexpr int TILES = Q / 16;
    static constexpr int NP = Q / 32;   // 32-token pairs
    // blocks of row tiles 0 .. I-1: ((I+1)/2)^2 for odd I, (I/2)(I/2+1) for
    // even I, written without a select (so that loads addressed with it stay
    // on straight-line code)
    static __host__ __device__ constexpr int off(int I) { return ((I >> 1) + 1) * ((I >> 1) + (I & 1)); }
    static constexpr int NBLK = off(TILES);
};

// Arguments of the decay-mask export kernel.
// Segsum evaluations of the mask export (the forward kernels use the first).
enum SegsumVariant : int {
    kSegsumHierarchy = 0,   // sub-block sums + rank-one off-diagonal factors
    kSegsumDirect = 1,      // every entry its own running sum, column by column
    kSegsumDiff = 2         // prefix sums over the chunk, entry = difference
};

struct MaskArgs {
    const float *dt;
    const float *A;
    const int32_t *seq_idx;
    float *out;          // [batch][nheads][count][Q][Q], nullable
    float *sums;         // [batch][nheads][count]: sum of each chunk's mask, nullable
    float *factors;      // [batch][nheads][count] SegRecords of the block-sum path, nullable
    int variant;         // SegsumVariant
    int batch, seqlen, nheads;
    int chunk_begin, count;
};

// Arguments of the single-token decode step.
struct DecodeArgs {
    const void *x;       // [batch][nheads][headdim]  (io dtype)
    const float *dt;     // [batch][nheads]
    const float *A;      // [nheads]
    const void *B;       // [batch][ngroups][dstate]  (io dtype)
    const void *C;       // [batch][ngroups][dstate]  (io dtype)
    const float *D;      // [nheads], nullable
    float *state;        // [batch][nheads][headdim][dstate], in/out
    void *y;             // [batch][nheads][headdim]  (io dtype)
    int batch, nheads, headdim, dstate, ngroups;
    // fused dt map and output gate, as in ChunkArgs (z: [batch][nheads][headdim])
    const float *dt_bias;
    const void *z;
    int dt_softplus, dt_clamp;
    float dt_lo, dt_hi;
};

// Arguments of the backward pass (fp32 gradients).
constexpr int kBwdQ = 64;   // tokens per backward chunk (= the states' split length)
struct BwdArgs {
    const void *x, *B, *C, *dy;       // io dtype
    const float *dt, *A, *D;          // D nullable
    const int32_t *seq_idx;           // nullable
    const float *states;              // [batch][nheads][nchunks][headdim][dstate] entering states,
                                      // nullable when there is one chunk
    const float *init_states;         // nullable
    const float *dfinal;              // nullable
    float *dx, *ddt;                  // [b][L][H][P], [b][L][H]
    float *dB_head, *dC_head;         // [b][L][H][N] workspace
    float *dA_part, *dD_part;         // [b][H][2] workspace (two slots per walk)
    float *dB, *dC, *dA, *dD, *dinit; // dD, dinit nullable
    int batch, seqlen, nheads, headdim, dstate, ngroups, nchunks;
    // The (batch row, head) walks whole_units .. whole_units + tail_units - 1
    // (the last, partial round of workgroups) run as two workgroups each:
    // chunks [split_chunk, nchunks) from dfinal, and chunks [0, split_chunk)
    // from g_tail[k] [headdim][dstate] fp32, the adjoint of the state at the
    // end of chunk split_chunk - 1, which the states kernel's extra workgroups
    // compute.  tail_units = 0: every walk whole.
    int whole_units, tail_units, split_chunk;
    float *g_tail;
};

struct Unit {
    int b, h, s, pb;
    int half;   // -1: the whole headdim block; 0 or 1: that half of it
};

// Workgroups are dealt to the 8 XCDs round-robin by block index.  Remap so
// that each XCD receives a contiguous range of logical units; logical units
// are ordered (batch, split, head, headdim block), so the heads of one batch
// row, and with sequence splits those of one split, which read the same
// per-group operands chunk by chunk, run on one XCD and share its L2
// (measured on the decay-stress workload, 16 heads x 16 splits: ordered
// (batch, head, split) every XCD walked all 256 chunks' operands, 838 MB of
// reads against 290 MB of algorithmic bytes).  Half units (the last,
// partial round of workgroups, two blocks each: halving them fills that
// round) are launched as a kernel of their own, whose block k is block
// whole + k here.  When the whole and the half units both divide by the 8
// XCDs, each XCD takes one contiguous range of units, the first part as
// whole units and the rest as half units: at the 2.7B layer one batch row,
// whose per-group operands its L2 then reads once (head kernels with the
// operands evicted from the caches: 195 -> 180 us; round-robin halves had
// made every XCD read the operands of both batch rows of that round, 70 MB
// of extra L2 misses).  Otherwise whole and half units are each dealt in
// contiguous ranges.
__device__ inline int xcd_contiguous(int blk, int count) {
    const int per = count / 8, rem = count % 8;
    const int xcd = blk % 8, k = blk / 8;
    return xcd * per + (xcd < rem ? xcd : rem) + k;
}

__device__ inline Unit unit_of_block(const ChunkArgs &a, int blk) {
    const int whole = a.units - a.half_units;
    int logical, half = -1;
    if (a.half_units > 0 && whole % 8 == 0 && a.half_units % 8 == 0) {
        // Each XCD takes one contiguous range of units, whole and half
        // alike: the first whole/8 of its range as whole units, the rest as
        // half units (at the 2.7B layer one batch row per XCD).
        const int per = a.units / 8, wper = whole / 8;
        if (blk < whole) {
            logical = (blk % 8) * per + blk / 8;
        } else {
            const int j = blk - whole, m = j / 8;
            logical = (j % 8) * per + wper + (m >> 1);
            half = m & 1;
        }
    } else if (blk < whole) {
        logical = xcd_contiguous(blk, whole);
    } else {
        const int j = xcd_contiguous(blk - whole, 2 * a.half_units);
        logical = whole + (j >> 1);
        half = j & 1;
    }
    Unit u;
    u.half = half;
    u.pb = logical % a.npblocks;
    int r = logical / a.npblocks;
    u.h = r % a.nheads;
    r /= a.nheads;
    u.s = r % a.nsplits;
    u.b = r / a.nsplits;
    return u;
}

__device__ inline float bf16_to_f32(bf16 v) { return (float)v; }

__device__ inline bf16x4 f32x4_to_bf16x4(f32x4 v) {
    bf16x4 r;
    r[0] = (bf16)v[0];
    r[1] = (bf16)v[1];
    r[2] = (bf16)v[2];
    r[3] = (bf16)v[3];
    return r;
}

// 16-bit transpose read from LDS (gfx950 ds_read_b64_tr_b16).  Within each
// group of 16 lanes, lane s supplies the address of 4 consecutive 16-bit
// elements; lane i of the group receives element (i % 4) of the loads made by
// lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4.  Callers point lane s at row
// (r0 + s/4), column (c0 + 4 (s % 4)) of a row-major tile, so lane i gets
// column c0 + i of rows r0 .. r0+3.
__device__ inline i16x4 lds_read_tr16(const bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
}

__device__ inline bf16x8 join_bf16x8(i16x4 lo, i16x4 hi) {
    i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// D = A B + C on v_mfma_f32_16x16x32_bf16.
__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A B.
__device__ inline f32x4 mfma_bf16_zero_acc(bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// MFMA results are not interlocked: on gfx950 a read of a
// v_mfma_f32_16x16x32_bf16 result needs 7 wait states (measured).  The
// compiler inserts them on straight-line code but has been seen to miss a read
// in the target block of a taken branch.  Values handed from MFMAs to vector
// code pass through here: the asm takes them as operands, so it sits after
// their MFMAs and before every read, on every path, and its s_nop supplies the
// wait states.  The build re-checks every path in the generated assembly.
__device__ inline void mfma_fence(f32x4 &a) { asm volatile("s_nop 7" : "+v"(a)); }
__device__ inline void mfma_fence(f32x4 &a, f32x4 &b) { asm volatile("s_nop 7" : "+v"(a), "+v"(b)); }

// The same for a whole array of accumulators (one wait for all of them).
template <int K>
__device__ inline void mfma_fence_all(f32x4 (&v)[K]) {
    asm volatile("s_nop 7" : "+v"(v[0]));
#pragma unroll
    for (int k = 1; k < K; ++k) asm volatile("" : "+v"(v[k]));
}

// The same for a two-dimensional array of accumulators.
template <int K1, int K2>
__device__ inline void mfma_fence_all(f32x4 (&v)[K1][K2]) {
    asm volatile("s_nop 7" : "+v"(v[0][0]));
#pragma unroll
    for (int i = 0; i < K1; ++i)
#pragma unroll
        for (int k = 0; k < K2; ++k)
            if (i + k > 0) asm volatile("" : "+v"(v[i][k]));
}

}  // namespace ssd
