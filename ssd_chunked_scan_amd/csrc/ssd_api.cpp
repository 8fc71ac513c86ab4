// Host side of the C ABI declared in include/ssd.h: argument validation,
// the split planner and the kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "ssd.h"
#include "ssd_common.hpp"

namespace ssd {
bool launch_scan_bf16_q64(int N, int PB, const ChunkArgs &a, hipStream_t stream);
bool launch_scan_bf16_q128(int N, int PB, const ChunkArgs &a, hipStream_t stream);
bool launch_scan_bf16_q256(int N, int PB, const ChunkArgs &a, hipStream_t stream);
bool launch_scan_bf16_direct(int N, int PB, const ChunkArgs &a, hipStream_t stream);
bool launch_scan_bf16_diff(int N, int PB, const ChunkArgs &a, hipStream_t stream);
bool launch_cb(int Q, int N, const CbArgs &a, hipStream_t stream);
size_t cb_s_elems(int Q);
void launch_chunk_f32(int Q, const ChunkArgs &a, hipStream_t stream);
void launch_bwd(bool bf16_io, const BwdArgs &a, hipStream_t stream);
void launch_bwd_states(bool bf16_io, const BwdArgs &a, float *out, hipStream_t stream);
void launch_split_scan(const float *init_states, float *ws_states, const float *ws_decay,
                       int batch, int nheads, int nsplits, int pn, hipStream_t stream);
void launch_mask(int Q, const MaskArgs &m, hipStream_t stream);
bool launch_decode(bool bf16_io, int N, const DecodeArgs &a, hipStream_t stream);
void launch_exp2_probe(uint32_t first, uint32_t count, uint32_t span, uint32_t *out, uint32_t nthreads,
                       hipStream_t stream);
void *noalloc_scratch(int dev, std::string *err);
}  // namespace ssd

namespace {

thread_local std::string g_last_error;

ssd_status_t fail(ssd_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool pow2_in(int64_t v, int64_t lo, int64_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

// Element counts above this are rejected so that every index fits the
// kernels' 64-bit offsets and every per-row count fits 32 bits.
constexpr int64_t kMaxDim = (int64_t)1 << 30;

ssd_status_t check_shape(const ssd_shape_t *s, int64_t chunk) {
    if (!s) return fail(SSD_ERR_NULL, "shape is NULL");
    if (s->batch < 1 || s->seqlen < 1 || s->nheads < 1 || s->headdim < 1 || s->dstate < 1 ||
        s->ngroups < 1)
        return fail(SSD_ERR_SHAPE, "sizes must be >= 1 (batch %lld seqlen %lld nheads %lld "
                    "headdim %lld dstate %lld ngroups %lld)", (long long)s->batch,
                    (long long)s->seqlen, (long long)s->nheads, (long long)s->headdim,
                    (long long)s->dstate, (long long)s->ngroups);
    if (s->nheads % s->ngroups != 0)
        return fail(SSD_ERR_SHAPE, "nheads (%lld) must be a multiple of ngroups (%lld)",
                    (long long)s->nheads, (long long)s->ngroups);
    if (s->batch > kMaxDim || s->seqlen > kMaxDim || s->nheads > 65536 ||
        s->batch * s->seqlen > kMaxDim)
        return fail(SSD_ERR_UNSUPPORTED, "problem too large");
    if (chunk != 64 && chunk != 128 && chunk != 256)
        return fail(SSD_ERR_UNSUPPORTED, "chunk_size %lld not in {64, 128, 256}", (long long)chunk);
    if (!pow2_in(s->headdim, 16, 128))
        return fail(SSD_ERR_UNSUPPORTED, "headdim %lld not in {16, 32, 64, 128}", (long long)s->headdim);
    if (!pow2_in(s->dstate, 16, 128))
        return fail(SSD_ERR_UNSUPPORTED, "dstate %lld not in {16, 32, 64, 128}", (long long)s->dstate);
    return SSD_OK;
}

int g_cu_cache[64];
std::atomic<int> g_cu_ready[64];

// Compute units of the device that `stream` belongs to (the current device
// for the null stream; cached per device; 256 when no device answers, so
// that planning also works in host-only tests).  The only HIP queries the
// planner makes.
int device_cus(hipStream_t stream) {
    int dev = -1;
    if (stream != nullptr) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
            (void)hipGetLastError();
            dev = -1;
        }
    }
    if (dev < 0 && hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < 0 || dev >= 64) return 256;
    if (g_cu_ready[dev].load(std::memory_order_acquire)) return g_cu_cache[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    g_cu_cache[dev] = cus;
    g_cu_ready[dev].store(1, std::memory_order_release);
    return cus;
}

// Workspace layout: the per-group operands first (their offsets depend only
// on the shape and the chunk size, so that a call with
// SSD_OPT_REUSE_GROUP_OPERANDS finds them whatever its split plan), then the
// split states and decays.
struct Plan {
    int nchunks, nsplits, split_chunks, npblocks, pblock, units, half_units;
    size_t s_bytes;       // per-group C B^T blocks (bf16)
    size_t bt_bytes;      // per-group token-transposed B (bf16)
    size_t c_bytes;       // per-group C in operand order (bf16)
    size_t split_bytes;   // split states + decays (nsplits > 1)
    size_t ws_bytes;
    size_t group_bytes() const { return s_bytes + bt_bytes + c_bytes; }
};

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Headdim block of the bf16 head kernel: the whole head, except at chunk 256
// with headdim 128, where the double-buffered X tile would not leave room
// (LDS and registers) -> two blocks of 64.
// LDS bytes of the bf16 head kernel for chunk Q, dstate N, headdim block PB:
// X stage, two fragment sets and the y tile (Q x PB bf16 each), the padded
// h^T tile and two buffers of segsum values.
int64_t bf16_lds_bytes(int64_t Q, int64_t N, int64_t PB) {
    const int64_t seg = 4 * (4 * Q + 2 * (Q / 16) + Q / 32);
    return 4 * Q * PB * 2 + PB * (N + 8) * 2 + 2 * seg;
}

// Units of the last, partial round of bf16 head-kernel workgroups, which run
// as two workgroups each (one per half of the headdim block): with W
// workgroups resident per device, U units take ceil(U / W) rounds and the last
// one holds T = U - (rounds - 1) W; when 2T <= W, halving those T units fills
// that round with workgroups of about half the work.
int bf16_half_units(int64_t units, int64_t Q, int64_t N, int64_t PB, int64_t cus) {
    if (PB < 32) return 0;
    const int64_t per_cu = std::max<int64_t>(1, (160 * 1024) / bf16_lds_bytes(Q, N, PB));
    const int64_t slots = cus * per_cu;
    const int64_t rounds = (units + slots - 1) / slots;
    const int64_t tail = units - (rounds - 1) * slots;
    return (rounds >= 2 && 2 * tail <= slots) ? (int)tail : 0;
}

// Largest headdim block (P, P/2, ...) whose workgroup fits in 160 KiB of LDS.
int bf16_pblock(int64_t Q, int64_t N, int64_t P) {
    int64_t pb = P;
    while (pb > 16 && bf16_lds_bytes(Q, N, pb) > 160 * 1024) pb /= 2;
    return (int)pb;
}

// Host-only validation of the problem description (no HIP call).
ssd_status_t check_problem(const ssd_shape_t *s, int64_t chunk, ssd_dtype_t io,
                           const ssd_options_t *opts) {
    if (io != SSD_F32 && io != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "unknown io dtype %d", (int)io);
    ssd_status_t st = check_shape(s, chunk);
    if (st != SSD_OK) return st;
    if (opts) {
        for (int k = 0; k < 5; ++k)
            if (opts->reserved[k] != 0) return fail(SSD_ERR_UNSUPPORTED, "reserved option fields must be zero");
        const int64_t hb = opts->headdim_block;
        if (hb != 0) {
            const bool pow2 = hb >= 16 && (hb & (hb - 1)) == 0;
            if (io == SSD_F32 ? hb != s->headdim
                              : (!pow2 || hb > s->headdim || s->headdim % hb != 0 ||
                                 bf16_lds_bytes(chunk, s->dstate, hb) > 160 * 1024))
                return fail(SSD_ERR_UNSUPPORTED, "headdim_block %lld is not usable for headdim %lld",
                            (long long)hb, (long long)s->headdim);
        }
        const int64_t known = SSD_OPT_REUSE_GROUP_OPERANDS | SSD_OPT_SEGSUM_DIRECT | SSD_OPT_SEGSUM_DIFF;
        if (opts->flags & ~known)
            return fail(SSD_ERR_UNSUPPORTED, "unknown option flags 0x%llx", (long long)opts->flags);
        const int64_t seg = opts->flags & (SSD_OPT_SEGSUM_DIRECT | SSD_OPT_SEGSUM_DIFF);
        if (seg == (SSD_OPT_SEGSUM_DIRECT | SSD_OPT_SEGSUM_DIFF))
            return fail(SSD_ERR_UNSUPPORTED, "segsum variants: one at a time");
        if (seg && io == SSD_BF16 && (chunk != 256 || (s->dstate != 64 && s->dstate != 128)))
            return fail(SSD_ERR_UNSUPPORTED, "bf16 segsum variants: chunk 256, dstate 64 or 128 only");
        if (opts->split_len < 0 || (opts->split_len > 0 && opts->split_len % chunk != 0))
            return fail(SSD_ERR_UNSUPPORTED, "split_len %lld must be 0 or a positive multiple of chunk_size",
                        (long long)opts->split_len);
    }
    return SSD_OK;
}

// Host-only validation of the fused prologue/epilogue block (NULL = none);
// z_align: required alignment of z in bytes.
ssd_status_t check_fused(const ssd_fused_t *fused, size_t z_align) {
    if (!fused) return SSD_OK;
    for (int k = 0; k < 4; ++k)
        if (fused->reserved[k] != 0) return fail(SSD_ERR_UNSUPPORTED, "reserved fused fields must be zero");
    if (fused->dt_clamp && !(std::isfinite(fused->dt_min) && std::isfinite(fused->dt_max) &&
                             fused->dt_min <= fused->dt_max))
        return fail(SSD_ERR_UNSUPPORTED, "dt clamp needs finite dt_min <= dt_max");
    if (fused->dt_bias && !aligned(fused->dt_bias, 4)) return fail(SSD_ERR_ALIGN, "dt_bias must be 4-byte aligned");
    if (fused->z && !aligned(fused->z, z_align))
        return fail(SSD_ERR_ALIGN, "z must be %zu-byte aligned", z_align);
    return SSD_OK;
}

// Largest grid (workgroups along x) any launch of the library may make.
constexpr int64_t kMaxGrid = 0x7fffffff;

// Split plan and workspace size of a validated problem; `stream` names the
// device whose compute-unit count the plan is made for.
ssd_status_t make_plan(const ssd_shape_t *s, int64_t chunk, ssd_dtype_t io,
                       const ssd_options_t *opts, Plan *pl, hipStream_t stream) {
    ssd_status_t st = check_problem(s, chunk, io, opts);
    if (st != SSD_OK) return st;
    pl->nchunks = (int)((s->seqlen + chunk - 1) / chunk);
    pl->pblock = (io == SSD_BF16) ? bf16_pblock(chunk, s->dstate, s->headdim) : (int)s->headdim;
    if (opts && opts->headdim_block > 0) pl->pblock = (int)opts->headdim_block;
    pl->npblocks = (int)(s->headdim / pl->pblock);
    int nsplits = 1;
    const int64_t cus = device_cus(stream);
    const bool forced_pb = opts && opts->headdim_block > 0;
    if (io == SSD_BF16 && !forced_pb && !(opts && opts->split_len > 0)) {
        // Too few (batch row, head) units for one workgroup per CU: halve the
        // headdim block first when that alone reaches a full round (no state
        // recomputation; measured on the 32-head sweep at 4 x 8192 tokens:
        // 166 us against 195 us for two sequence splits).
        const int64_t units = s->batch * s->nheads * pl->npblocks;
        if (units < cus && 2 * units >= cus && pl->pblock >= 64) {
            pl->pblock /= 2;
            pl->npblocks *= 2;
        }
    }
    if (opts && opts->split_len > 0) {
        const int64_t sc = opts->split_len / chunk;
        nsplits = (int)((pl->nchunks + sc - 1) / sc);
    } else {
        // Split-sequence planning: the split length is chosen from the amount
        // of independent work, not from the chunk size.  Enough splits for
        // one round of workgroups over the CUs (a second round costs more in
        // per-workgroup start-up and in the split-local pass than it gains:
        // measured 4096-token splits 189-200 us against 2048-token splits
        // 213-270 us at 2 x 16384 x 32 heads and 1 x 65536 x 16 heads); rows
        // never split below one chunk per split.
        const int64_t units = s->batch * s->nheads * pl->npblocks;
        if (units < cus) {
            const int64_t want = (cus + units - 1) / units;
            nsplits = (int)std::min<int64_t>(want, pl->nchunks);
        }
    }
    pl->split_chunks = (pl->nchunks + nsplits - 1) / nsplits;
    pl->nsplits = (pl->nchunks + pl->split_chunks - 1) / pl->split_chunks;
    // Every grid must fit the launch limit and every unit index an int.
    const int64_t units = s->batch * s->nheads * (int64_t)pl->nsplits * pl->npblocks;
    if (units > kMaxGrid / 2 || s->batch * s->nheads > kMaxGrid / 2 ||
        s->batch * s->ngroups * (int64_t)pl->nchunks * (chunk / 64) > kMaxGrid)
        return fail(SSD_ERR_UNSUPPORTED, "problem too large: %lld work units", (long long)units);
    pl->units = (int)units;
    pl->half_units = (io == SSD_BF16) ? bf16_half_units(units, chunk, s->dstate, pl->pblock, cus) : 0;
    if (io == SSD_BF16 && opts && (opts->flags & (SSD_OPT_SEGSUM_DIRECT | SSD_OPT_SEGSUM_DIFF)) &&
        pl->pblock != 32 && pl->pblock != 64)
        return fail(SSD_ERR_UNSUPPORTED, "bf16 segsum variants: headdim blocks of 32 or 64 only (planned %d)",
                    pl->pblock);
    pl->split_bytes = 0;
    if (pl->nsplits > 1) {
        const size_t states = (size_t)s->batch * s->nheads * pl->nsplits * s->headdim * s->dstate;
        const size_t decay = (size_t)s->batch * s->nheads * pl->nsplits;
        pl->split_bytes = round_up((states + decay) * sizeof(float), 256);
    }
    pl->s_bytes = pl->bt_bytes = pl->c_bytes = 0;
    if (io == SSD_BF16) {
        const size_t bgc = (size_t)s->batch * s->ngroups * pl->nchunks;
        pl->s_bytes = round_up(bgc * ssd::cb_s_elems((int)chunk) * 2, 256);
        pl->bt_bytes = round_up(bgc * (size_t)chunk * s->dstate * 2, 256);
        pl->c_bytes = round_up(bgc * (size_t)chunk * std::max<int64_t>(s->dstate, 32) * 2, 256);
    }
    pl->ws_bytes = pl->group_bytes() + pl->split_bytes;
    return SSD_OK;
}

}  // namespace

extern "C" {

const char *ssd_status_str(ssd_status_t status) {
    switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
    case SSD_ERR_HIP: return "SSD_ERR_HIP";
    }
    return "SSD_ERR_UNKNOWN";
}

const char *ssd_last_error(void) { return g_last_error.c_str(); }

const char *ssd_version(void) { return "ssd-mi355x 0.1 (gfx950)"; }

size_t ssd_fwd_ex_workspace_bytes(const ssd_shape_t *shape, int64_t chunk_size, ssd_dtype_t io,
                                  const ssd_options_t *opts) {
    Plan pl;
    if (make_plan(shape, chunk_size, io, opts, &pl, nullptr) != SSD_OK) return 0;
    return pl.ws_bytes;
}

size_t ssd_fwd_workspace_bytes(const ssd_shape_t *shape, int64_t chunk_size, ssd_dtype_t io) {
    return ssd_fwd_ex_workspace_bytes(shape, chunk_size, io, nullptr);
}

int64_t ssd_plan_split_len(const ssd_shape_t *shape, int64_t chunk_size, ssd_dtype_t io) {
    Plan pl;
    if (make_plan(shape, chunk_size, io, nullptr, &pl, nullptr) != SSD_OK) return 0;
    return (int64_t)pl.split_chunks * chunk_size;
}

int64_t ssd_plan_headdim_block(const ssd_shape_t *shape, int64_t chunk_size, ssd_dtype_t io) {
    Plan pl;
    if (make_plan(shape, chunk_size, io, nullptr, &pl, nullptr) != SSD_OK) return 0;
    return pl.pblock;
}

}  // extern "C"

namespace {

// The forward pass; with states_only, only what gives every split its
// entering state (per-group operands, split-local pass, affine scan): the
// outputs are not computed and y may be NULL (the backward pass uses this
// with one split per chunk).  dbg_seg (bf16 io, nullable): the head kernel
// also writes each chunk's segsum factors there.
ssd_status_t fwd_impl(const ssd_shape_t *shape, ssd_dtype_t io, const void *x, const float *dt,
                      const float *A, const void *B, const void *C, const float *D,
                      const int32_t *seq_idx, int64_t chunk_size, const float *init_states,
                      void *y, float *final_states, const ssd_fused_t *fused,
                      void *workspace, size_t workspace_bytes, const ssd_options_t *opts,
                      void *stream, bool states_only, float *dbg_seg = nullptr,
                      bool validate_only = false) {
    ssd_status_t st = check_problem(shape, chunk_size, io, opts);
    if (st != SSD_OK) return st;
    st = check_fused(fused, 16);
    if (st != SSD_OK) return st;
    if (!x || !dt || !A || !B || !C || (!y && !states_only))
        return fail(SSD_ERR_NULL, "x, dt, A, B, C and y are required");
    const size_t io_align = 16;
    if (!aligned(x, io_align) || !aligned(B, io_align) || !aligned(C, io_align) || (y && !aligned(y, io_align)))
        return fail(SSD_ERR_ALIGN, "x, B, C and y must be 16-byte aligned");
    if (!aligned(dt, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) || (seq_idx && !aligned(seq_idx, 4)))
        return fail(SSD_ERR_ALIGN, "dt, A, D and seq_idx must be 4-byte aligned");
    if ((init_states && !aligned(init_states, 16)) || (final_states && !aligned(final_states, 16)))
        return fail(SSD_ERR_ALIGN, "init_states and final_states must be 16-byte aligned");
    if (workspace && !aligned(workspace, 16)) return fail(SSD_ERR_ALIGN, "workspace must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    Plan pl;
    st = make_plan(shape, chunk_size, io, opts, &pl, s);
    if (st != SSD_OK) return st;
    if (validate_only) return SSD_OK;
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes))
        return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given%s", pl.ws_bytes,
                    workspace_bytes, workspace ? "" : " (NULL)");

    ssd::ChunkArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.seq_idx = seq_idx;
    a.init_states = init_states;
    a.y = y;
    a.final_states = final_states;
    char *wsb = (char *)workspace;
    a.ws_S = pl.s_bytes ? wsb : nullptr;
    a.ws_BT = pl.bt_bytes ? wsb + pl.s_bytes : nullptr;
    a.ws_C = pl.c_bytes ? wsb + pl.s_bytes + pl.bt_bytes : nullptr;
    float *ws_split = pl.nsplits > 1 ? (float *)(wsb + pl.group_bytes()) : nullptr;
    a.ws_states = ws_split;
    a.ws_decay = pl.nsplits > 1
                     ? ws_split + (size_t)shape->batch * shape->nheads * pl.nsplits * shape->headdim * shape->dstate
                     : nullptr;
    a.batch = (int)shape->batch;
    a.seqlen = (int)shape->seqlen;
    a.nheads = (int)shape->nheads;
    a.headdim = (int)shape->headdim;
    a.dstate = (int)shape->dstate;
    a.ngroups = (int)shape->ngroups;
    a.chunk = (int)chunk_size;
    a.nchunks = pl.nchunks;
    a.nsplits = pl.nsplits;
    a.split_chunks = pl.split_chunks;
    a.npblocks = pl.npblocks;
    a.pblock = pl.pblock;
    a.units = pl.units;
    a.half_units = pl.half_units;
    a.dbg_seg = dbg_seg;
    if (opts && (opts->flags & SSD_OPT_SEGSUM_DIRECT)) a.segsum_variant = ssd::kSegsumDirect;
    if (opts && (opts->flags & SSD_OPT_SEGSUM_DIFF)) a.segsum_variant = ssd::kSegsumDiff;
    if (fused) {
        a.dt_bias = fused->dt_bias;
        a.z = fused->z;
        a.dt_softplus = fused->dt_softplus != 0;
        a.dt_clamp = fused->dt_clamp != 0;
        a.dt_lo = fused->dt_min;
        a.dt_hi = fused->dt_max;
    }

    auto launch = [&](const ssd::ChunkArgs &args) -> bool {
        if (io == SSD_F32) {
            ssd::launch_chunk_f32(args.chunk, args, s);
            return true;
        }
        if (args.mode == ssd::kModeFull && args.segsum_variant == ssd::kSegsumDirect)
            return ssd::launch_scan_bf16_direct(args.dstate, args.pblock, args, s);
        if (args.mode == ssd::kModeFull && args.segsum_variant == ssd::kSegsumDiff)
            return ssd::launch_scan_bf16_diff(args.dstate, args.pblock, args, s);
        switch (args.chunk) {
        case 64: return ssd::launch_scan_bf16_q64(args.dstate, args.pblock, args, s);
        case 128: return ssd::launch_scan_bf16_q128(args.dstate, args.pblock, args, s);
        default: return ssd::launch_scan_bf16_q256(args.dstate, args.pblock, args, s);
        }
    };

    (void)hipGetLastError();
    const bool reuse = opts && (opts->flags & SSD_OPT_REUSE_GROUP_OPERANDS);
    if (io == SSD_BF16 && !reuse) {
        ssd::CbArgs cb;
        memset(&cb, 0, sizeof(cb));
        cb.B = B;
        cb.C = C;
        cb.ws_S = wsb;
        cb.ws_BT = wsb + pl.s_bytes;
        cb.ws_C = wsb + pl.s_bytes + pl.bt_bytes;
        cb.batch = a.batch;
        cb.seqlen = a.seqlen;
        cb.ngroups = a.ngroups;
        cb.nchunks = a.nchunks;
        if (!ssd::launch_cb(a.chunk, a.dstate, cb, s)) return fail(SSD_ERR_UNSUPPORTED, "no C B^T kernel for this shape");
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SSD_ERR_HIP, "C B^T launch: %s", hipGetErrorString(e));
    }
    if (a.nsplits > 1) {
        ssd::ChunkArgs loc = a;
        loc.mode = ssd::kModeSplitLocal;
        if (!launch(loc)) return fail(SSD_ERR_UNSUPPORTED, "no kernel for this shape");
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SSD_ERR_HIP, "split-local launch: %s", hipGetErrorString(e));
        ssd::launch_split_scan(init_states, a.ws_states, a.ws_decay, a.batch, a.nheads, a.nsplits,
                               a.headdim * a.dstate, s);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(SSD_ERR_HIP, "split-scan launch: %s", hipGetErrorString(e));
    }
    if (states_only) return SSD_OK;
    a.mode = ssd::kModeFull;
    if (!launch(a)) return fail(SSD_ERR_UNSUPPORTED, "no kernel for this shape");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "chunk launch: %s", hipGetErrorString(e));
    return SSD_OK;
}

// Backward workspace: the chunk-entering states (when there is more than
// one 64-token chunk), then the per-head dB and dC, the dA and dD partial
// sums (two slots per walk) and the adjoints the tail walks start from.
//
// Tail split: the reverse walks are one workgroup per (batch row, head), one
// per compute unit.  When they outnumber the CUs and the last round holds at
// most half of them, each walk of that round runs as two workgroups over
// half the chunks each, the earlier half starting from an adjoint computed
// beforehand (by the states kernel, alongside the states): the last round
// then takes about half as long.
struct BwdPlan {
    Plan fwd;
    int whole_units, tail_units, split_chunk;
    size_t states_bytes, dbh_bytes, part_bytes, tail_bytes, ws_bytes;
};

ssd_status_t make_bwd_plan(const ssd_shape_t *s, ssd_dtype_t io, BwdPlan *bp, hipStream_t stream) {
    ssd_options_t o;
    memset(&o, 0, sizeof(o));
    o.split_len = ssd::kBwdQ;
    ssd_status_t st = make_plan(s, ssd::kBwdQ, io, &o, &bp->fwd, stream);
    if (st != SSD_OK) return st;
    bp->states_bytes = bp->fwd.nchunks > 1
                           ? round_up((size_t)s->batch * s->nheads * bp->fwd.nchunks * s->headdim *
                                          s->dstate * sizeof(float), 256)
                           : 0;
    bp->dbh_bytes = round_up((size_t)s->batch * s->seqlen * s->nheads * s->dstate * sizeof(float), 256);
    bp->part_bytes = round_up((size_t)s->batch * s->nheads * 2 * sizeof(float), 256);
    const int64_t units = s->batch * s->nheads, cus = device_cus(stream);
    const int64_t tail = units % cus;
    const bool split = units > cus && tail > 0 && 2 * tail <= cus && bp->fwd.nchunks >= 2;
    bp->tail_units = split ? (int)tail : 0;
    bp->whole_units = (int)(units - bp->tail_units);
    bp->split_chunk = bp->fwd.nchunks / 2;
    bp->tail_bytes = round_up((size_t)bp->tail_units * s->headdim * s->dstate * sizeof(float), 256);
    bp->ws_bytes = bp->states_bytes + 2 * bp->dbh_bytes + 2 * bp->part_bytes + bp->tail_bytes;
    return SSD_OK;
}

}  // namespace

extern "C" {

ssd_status_t ssd_fwd_fused(const ssd_shape_t *shape, ssd_dtype_t io, const void *x, const float *dt,
                           const float *A, const void *B, const void *C, const float *D,
                           const int32_t *seq_idx, int64_t chunk_size, const float *init_states,
                           void *y, float *final_states, const ssd_fused_t *fused,
                           void *workspace, size_t workspace_bytes, const ssd_options_t *opts,
                           void *stream) {
    g_last_error.clear();
    return fwd_impl(shape, io, x, dt, A, B, C, D, seq_idx, chunk_size, init_states, y, final_states,
                    fused, workspace, workspace_bytes, opts, stream, false);
}

size_t ssd_bwd_workspace_bytes(const ssd_shape_t *shape, ssd_dtype_t io) {
    BwdPlan bp;
    if (make_bwd_plan(shape, io, &bp, nullptr) != SSD_OK) return 0;
    return bp.ws_bytes;
}

ssd_status_t ssd_bwd(const ssd_shape_t *shape, ssd_dtype_t io, const void *x, const float *dt,
                     const float *A, const void *B, const void *C, const float *D,
                     const int32_t *seq_idx, const float *init_states, const void *dy,
                     const float *dfinal, float *dx, float *ddt, float *dA, float *dB, float *dC,
                     float *dD, float *dinit, void *workspace, size_t workspace_bytes,
                     void *stream) {
    g_last_error.clear();
    BwdPlan bp;
    ssd_status_t st = make_bwd_plan(shape, io, &bp, (hipStream_t)stream);
    if (st != SSD_OK) return st;
    if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC)
        return fail(SSD_ERR_NULL, "x, dt, A, B, C, dy, dx, ddt, dA, dB and dC are required");
    if ((D == nullptr) != (dD == nullptr)) return fail(SSD_ERR_NULL, "D and dD go together");
    if (dinit && !init_states) return fail(SSD_ERR_NULL, "dinit needs init_states");
    const size_t esz = io == SSD_BF16 ? 2 : 4;
    if (!aligned(dy, 16)) return fail(SSD_ERR_ALIGN, "dy must be 16-byte aligned");
    if (!aligned(dx, 4) || !aligned(ddt, 4) || !aligned(dA, 4) || !aligned(dB, 4) || !aligned(dC, 4) ||
        (dD && !aligned(dD, 4)) || (dinit && !aligned(dinit, 4)) || (dfinal && !aligned(dfinal, 4)))
        return fail(SSD_ERR_ALIGN, "gradient buffers and dfinal must be 4-byte aligned");
    (void)esz;
    if (!workspace || workspace_bytes < bp.ws_bytes)
        return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given%s", bp.ws_bytes,
                    workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 16)) return fail(SSD_ERR_ALIGN, "workspace must be 16-byte aligned");
    // the gradient reduction runs one thread per (row, token, group, state) element
    if ((shape->batch * shape->seqlen * shape->ngroups * shape->dstate + shape->nheads) / 256 >= kMaxGrid)
        return fail(SSD_ERR_UNSUPPORTED, "problem too large for the gradient reduction grid");
    ssd_options_t o;
    memset(&o, 0, sizeof(o));
    o.split_len = ssd::kBwdQ;
    // the forward's checks of the shared inputs (nothing is launched)
    st = fwd_impl(shape, io, x, dt, A, B, C, D, seq_idx, ssd::kBwdQ, init_states, nullptr, nullptr,
                  nullptr, nullptr, 0, &o, stream, true, nullptr, true);
    if (st != SSD_OK) return st;
    char *wsb = (char *)workspace + bp.states_bytes;
    ssd::BwdArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x;
    a.B = B;
    a.C = C;
    a.dy = dy;
    a.dt = dt;
    a.A = A;
    a.D = D;
    a.seq_idx = seq_idx;
    float *states = bp.states_bytes ? (float *)workspace : nullptr;
    a.states = states;
    a.init_states = init_states;
    a.dfinal = dfinal;
    a.dx = dx;
    a.ddt = ddt;
    a.dB_head = (float *)wsb;
    a.dC_head = (float *)(wsb + bp.dbh_bytes);
    a.dA_part = (float *)(wsb + 2 * bp.dbh_bytes);
    a.dD_part = (float *)(wsb + 2 * bp.dbh_bytes + bp.part_bytes);
    a.g_tail = bp.tail_units ? (float *)(wsb + 2 * bp.dbh_bytes + 2 * bp.part_bytes) : nullptr;
    a.whole_units = bp.whole_units;
    a.tail_units = bp.tail_units;
    a.split_chunk = bp.split_chunk;
    a.dB = dB;
    a.dC = dC;
    a.dA = dA;
    a.dD = dD;
    a.dinit = dinit;
    a.batch = (int)shape->batch;
    a.seqlen = (int)shape->seqlen;
    a.nheads = (int)shape->nheads;
    a.headdim = (int)shape->headdim;
    a.dstate = (int)shape->dstate;
    a.ngroups = (int)shape->ngroups;
    a.nchunks = bp.fwd.nchunks;
    (void)hipGetLastError();
    if (states) {   // H_{c-1} of every chunk, walked in order
        ssd::launch_bwd_states(io == SSD_BF16, a, states, (hipStream_t)stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SSD_ERR_HIP, "backward states launch: %s", hipGetErrorString(e));
    }
    ssd::launch_bwd(io == SSD_BF16, a, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return SSD_OK;
}

ssd_status_t ssd_fwd_ex(const ssd_shape_t *shape, ssd_dtype_t io, const void *x, const float *dt,
                        const float *A, const void *B, const void *C, const float *D,
                        const int32_t *seq_idx, int64_t chunk_size, const float *init_states,
                        void *y, float *final_states, void *workspace, size_t workspace_bytes,
                        const ssd_options_t *opts, void *stream) {
    return ssd_fwd_fused(shape, io, x, dt, A, B, C, D, seq_idx, chunk_size, init_states, y,
                         final_states, nullptr, workspace, workspace_bytes, opts, stream);
}

ssd_status_t ssd_fwd(const ssd_shape_t *shape, ssd_dtype_t io, const void *x, const float *dt,
                     const float *A, const void *B, const void *C, const float *D,
                     const int32_t *seq_idx, int64_t chunk_size, const float *init_states, void *y,
                     float *final_states, void *workspace, size_t workspace_bytes, void *stream) {
    return ssd_fwd_ex(shape, io, x, dt, A, B, C, D, seq_idx, chunk_size, init_states, y, final_states,
                      workspace, workspace_bytes, nullptr, stream);
}

ssd_status_t ssd_debug_chunk_mask(const ssd_shape_t *shape, const float *dt, const float *A,
                                  const int32_t *seq_idx, int64_t chunk_size, int64_t chunk_begin,
                                  int64_t chunk_count, float *L_out, void *stream) {
    if (!L_out) {
        g_last_error.clear();
        return fail(SSD_ERR_NULL, "L_out is required");
    }
    return ssd_debug_chunk_mask_ex(shape, dt, A, seq_idx, chunk_size, chunk_begin, chunk_count,
                                   SSD_SEGSUM_HIERARCHY, L_out, nullptr, stream);
}

ssd_status_t ssd_debug_chunk_mask_ex(const ssd_shape_t *shape, const float *dt, const float *A,
                                     const int32_t *seq_idx, int64_t chunk_size, int64_t chunk_begin,
                                     int64_t chunk_count, int32_t variant, float *L_out,
                                     float *sums_out, void *stream) {
    g_last_error.clear();
    ssd_status_t st = check_shape(shape, chunk_size);
    if (st != SSD_OK) return st;
    if (!dt || !A) return fail(SSD_ERR_NULL, "dt and A are required");
    if (!L_out && !sums_out) return fail(SSD_ERR_NULL, "at least one of L_out and sums_out is required");
    if (variant != SSD_SEGSUM_HIERARCHY && variant != SSD_SEGSUM_DIRECT && variant != SSD_SEGSUM_DIFF)
        return fail(SSD_ERR_UNSUPPORTED, "unknown segsum variant %d", (int)variant);
    if (L_out && !aligned(L_out, 16)) return fail(SSD_ERR_ALIGN, "L_out must be 16-byte aligned");
    if (sums_out && !aligned(sums_out, 4)) return fail(SSD_ERR_ALIGN, "sums_out must be 4-byte aligned");
    if (!aligned(dt, 4) || !aligned(A, 4) || (seq_idx && !aligned(seq_idx, 4)))
        return fail(SSD_ERR_ALIGN, "dt, A and seq_idx must be 4-byte aligned");
    const int64_t nchunks = (shape->seqlen + chunk_size - 1) / chunk_size;
    if (chunk_begin < 0 || chunk_count < 1 || chunk_begin + chunk_count > nchunks || chunk_count > 65535)
        return fail(SSD_ERR_SHAPE, "chunk range [%lld, %lld) outside [0, %lld)", (long long)chunk_begin,
                    (long long)(chunk_begin + chunk_count), (long long)nchunks);
    ssd::MaskArgs m;
    memset(&m, 0, sizeof(m));   // every field not set below (factors) stays null
    m.dt = dt;
    m.A = A;
    m.seq_idx = seq_idx;
    m.out = L_out;
    m.sums = sums_out;
    m.variant = (int)variant;
    m.batch = (int)shape->batch;
    m.seqlen = (int)shape->seqlen;
    m.nheads = (int)shape->nheads;
    m.chunk_begin = (int)chunk_begin;
    m.count = (int)chunk_count;
    (void)hipGetLastError();
    ssd::launch_mask((int)chunk_size, m, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "mask launch: %s", hipGetErrorString(e));
    return SSD_OK;
}

ssd_status_t ssd_decode_step(const ssd_shape_t *shape, ssd_dtype_t io, const void *x,
                             const float *dt, const float *A, const void *B, const void *C,
                             const float *D, float *state, void *y, void *stream) {
    return ssd_decode_step_fused(shape, io, x, dt, A, B, C, D, state, y, nullptr, stream);
}

ssd_status_t ssd_decode_step_fused(const ssd_shape_t *shape, ssd_dtype_t io, const void *x,
                                   const float *dt, const float *A, const void *B, const void *C,
                                   const float *D, float *state, void *y, const ssd_fused_t *fused,
                                   void *stream) {
    g_last_error.clear();
    if (io != SSD_F32 && io != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "unknown io dtype %d", (int)io);
    ssd_status_t st = check_shape(shape, 64);
    if (st != SSD_OK) return st;
    if (shape->seqlen != 1) return fail(SSD_ERR_SHAPE, "a decode step takes one token (seqlen %lld)",
                                        (long long)shape->seqlen);
    if (shape->batch * shape->nheads > kMaxGrid)
        return fail(SSD_ERR_UNSUPPORTED, "batch * nheads above the launch limit");
    if (!x || !dt || !A || !B || !C || !state || !y)
        return fail(SSD_ERR_NULL, "x, dt, A, B, C, state and y are required");
    const size_t esz = io == SSD_BF16 ? 2 : 4;
    if (!aligned(x, esz) || !aligned(B, esz) || !aligned(C, esz) || !aligned(y, esz))
        return fail(SSD_ERR_ALIGN, "x, B, C and y must be aligned to their element size");
    if (!aligned(dt, 4) || !aligned(A, 4) || (D && !aligned(D, 4)))
        return fail(SSD_ERR_ALIGN, "dt, A and D must be 4-byte aligned");
    if (!aligned(state, 16)) return fail(SSD_ERR_ALIGN, "state must be 16-byte aligned");
    st = check_fused(fused, esz);
    if (st != SSD_OK) return st;
    ssd::DecodeArgs a;
    memset(&a, 0, sizeof(a));
    if (fused) {
        a.dt_bias = fused->dt_bias;
        a.z = fused->z;
        a.dt_softplus = fused->dt_softplus != 0;
        a.dt_clamp = fused->dt_clamp != 0;
        a.dt_lo = fused->dt_min;
        a.dt_hi = fused->dt_max;
    }
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.state = state;
    a.y = y;
    a.batch = (int)shape->batch;
    a.nheads = (int)shape->nheads;
    a.headdim = (int)shape->headdim;
    a.dstate = (int)shape->dstate;
    a.ngroups = (int)shape->ngroups;
    (void)hipGetLastError();
    if (!ssd::launch_decode(io == SSD_BF16, a.dstate, a, (hipStream_t)stream))
        return fail(SSD_ERR_UNSUPPORTED, "no decode kernel for dstate %d", a.dstate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return SSD_OK;
}


ssd_status_t ssd_fwd_noalloc(const ssd_shape_t *shape, ssd_dtype_t io, const void *x, const float *dt,
                             const float *A, const void *B, const void *C, const float *D,
                             const int32_t *seq_idx, int64_t chunk_size, const float *init_states,
                             void *y, float *final_states, void *stream) {
    g_last_error.clear();
    ssd_status_t st = check_problem(shape, chunk_size, io, nullptr);
    if (st != SSD_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    Plan pl;
    st = make_plan(shape, chunk_size, io, nullptr, &pl, s);
    if (st != SSD_OK) return st;
    if (pl.ws_bytes > SSD_NOALLOC_WORKSPACE_BYTES)
        return fail(SSD_ERR_WORKSPACE, "ssd_fwd_noalloc: this problem needs %zu bytes of workspace, "
                    "above the fixed %zu bytes; use ssd_fwd with a caller-allocated workspace",
                    pl.ws_bytes, (size_t)SSD_NOALLOC_WORKSPACE_BYTES);
    void *ws = nullptr;
    if (pl.ws_bytes > 0) {
        int dev = -1;
        if (s == nullptr || hipStreamGetDevice(s, &dev) != hipSuccess) {
            (void)hipGetLastError();
            if (hipGetDevice(&dev) != hipSuccess) {
                (void)hipGetLastError();
                return fail(SSD_ERR_HIP, "no current device");
            }
        }
        std::string err;
        ws = ssd::noalloc_scratch(dev, &err);
        if (!ws) return fail(SSD_ERR_HIP, "%s", err.c_str());
    }
    return fwd_impl(shape, io, x, dt, A, B, C, D, seq_idx, chunk_size, init_states, y, final_states,
                    nullptr, ws, ws ? (size_t)SSD_NOALLOC_WORKSPACE_BYTES : 0, nullptr, stream, false);
}

int64_t ssd_segsum_record_words(int64_t chunk_size) {
    if (chunk_size != 64 && chunk_size != 128 && chunk_size != 256) return 0;
    return 4 * chunk_size + 2 * (chunk_size / 16) + chunk_size / 32;
}

ssd_status_t ssd_debug_segsum_factors(const ssd_shape_t *shape, const float *dt, const float *A,
                                      const int32_t *seq_idx, int64_t chunk_size, float *out,
                                      void *stream) {
    g_last_error.clear();
    ssd_status_t st = check_shape(shape, chunk_size);
    if (st != SSD_OK) return st;
    if (!dt || !A || !out) return fail(SSD_ERR_NULL, "dt, A and out are required");
    if (!aligned(dt, 4) || !aligned(A, 4) || (seq_idx && !aligned(seq_idx, 4)) || !aligned(out, 4))
        return fail(SSD_ERR_ALIGN, "dt, A, seq_idx and out must be 4-byte aligned");
    const int64_t nchunks = (shape->seqlen + chunk_size - 1) / chunk_size;
    if (nchunks > 65535) return fail(SSD_ERR_UNSUPPORTED, "more than 65535 chunks");
    ssd::MaskArgs m;
    memset(&m, 0, sizeof(m));
    m.dt = dt;
    m.A = A;
    m.seq_idx = seq_idx;
    m.factors = out;
    m.variant = SSD_SEGSUM_HIERARCHY;
    m.batch = (int)shape->batch;
    m.seqlen = (int)shape->seqlen;
    m.nheads = (int)shape->nheads;
    m.chunk_begin = 0;
    m.count = (int)nchunks;
    (void)hipGetLastError();
    ssd::launch_mask((int)chunk_size, m, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "segsum factor launch: %s", hipGetErrorString(e));
    return SSD_OK;
}

ssd_status_t ssd_debug_fwd_segsum_factors(const ssd_shape_t *shape, ssd_dtype_t io, const void *x,
                                          const float *dt, const float *A, const void *B,
                                          const void *C, const float *D, const int32_t *seq_idx,
                                          int64_t chunk_size, const float *init_states, void *y,
                                          float *final_states, void *workspace,
                                          size_t workspace_bytes, const ssd_options_t *opts,
                                          float *out, void *stream) {
    g_last_error.clear();
    if (io != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "the segsum factor export is a bf16-path debug aid");
    if (!out) return fail(SSD_ERR_NULL, "out is required");
    if (!aligned(out, 4)) return fail(SSD_ERR_ALIGN, "out must be 4-byte aligned");
    return fwd_impl(shape, io, x, dt, A, B, C, D, seq_idx, chunk_size, init_states, y, final_states,
                    nullptr, workspace, workspace_bytes, opts, stream, false, out);
}

ssd_status_t ssd_debug_exp2_probe(uint32_t first_bits, uint32_t count, uint32_t *counts,
                                  uint32_t nthreads, void *stream) {
    g_last_error.clear();
    if (!counts) return fail(SSD_ERR_NULL, "counts is required");
    if (!aligned(counts, 4)) return fail(SSD_ERR_ALIGN, "counts must be 4-byte aligned");
    if (first_bits < 0x80000000u || count == 0 || (uint64_t)first_bits + count - 1 > 0xFF800000u)
        return fail(SSD_ERR_UNSUPPORTED, "the probe covers non-positive fp32 patterns in "
                    "[0x80000000, 0xff800000] (-0 .. -inf)");
    if (nthreads == 0 || nthreads > (1u << 24)) return fail(SSD_ERR_UNSUPPORTED, "nthreads must be in [1, 2^24]");
    const uint32_t span = (uint32_t)(((uint64_t)count + nthreads - 1) / nthreads);
    (void)hipGetLastError();
    ssd::launch_exp2_probe(first_bits, count, span, counts, nthreads, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "exp2 probe launch: %s", hipGetErrorString(e));
    return SSD_OK;
}

}  // extern "C"
