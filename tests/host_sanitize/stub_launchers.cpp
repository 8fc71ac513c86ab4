// Host stand-ins for the kernel launchers of libssd, for the sanitizer build
// of the C ABI's host code (ssd_api.cpp).  Each stub reads every byte of
// every buffer the real kernel reads and writes every byte it writes, with
// the extents derived from the launch arguments the way the kernels index
// them.  The driver passes host buffers of exactly the documented sizes, so
// AddressSanitizer reports any launch whose arguments would reach outside a
// caller's buffer or outside the workspace.
#include <cstdint>
#include <cstring>
#include <string>

#include "ssd.h"

#include "ssd_common.hpp"

namespace {

volatile uint64_t g_sink;
uint64_t g_launches;

void rd(const void *p, size_t n) {
    if (!p || n == 0) return;
    const unsigned char *c = (const unsigned char *)p;
    uint64_t s = 0;
    for (size_t k = 0; k < n; ++k) s += c[k];
    g_sink = g_sink + s;
}

void wr(void *p, size_t n) {
    if (p && n) memset(p, 0x5a, n);
}

size_t nblk(int Q) {
    const int t = Q / 16;
    return (size_t)(t / 2) * (t / 2 + 1);
}

void group_operands(const ssd::ChunkArgs &a, bool write) {
    const size_t bgc = (size_t)a.batch * a.ngroups * a.nchunks;
    const int Q = a.chunk, N = a.dstate, KN = N >= 32 ? N / 32 : 1;
    const size_t s = bgc * nblk(Q) * 64 * 16, bt = bgc * (Q / 32) * N * 4 * 16,
                 c = bgc * (Q / 16) * KN * 64 * 16;
    if (write) {
        wr((void *)a.ws_S, s);
        wr((void *)a.ws_BT, bt);
        wr((void *)a.ws_C, c);
    } else {
        rd(a.ws_S, s);
        rd(a.ws_BT, bt);
        rd(a.ws_C, c);
    }
}

void chunk_pass(const ssd::ChunkArgs &a, size_t esz) {
    ++g_launches;
    const size_t b = a.batch, L = a.seqlen, H = a.nheads, P = a.headdim, N = a.dstate, G = a.ngroups;
    rd(a.x, b * L * H * P * esz);
    rd(a.dt, b * L * H * 4);
    rd(a.A, H * 4);
    rd(a.D, a.D ? H * 4 : 0);
    rd(a.seq_idx, a.seq_idx ? b * L * 4 : 0);
    rd(a.dt_bias, a.dt_bias ? H * 4 : 0);
    if (esz == 2) group_operands(a, false);
    if (a.mode == ssd::kModeSplitLocal) {
        wr(a.ws_states, b * H * (a.nsplits - 1) * P * N * 4);   // the last split keeps no summary
        wr(a.ws_decay, b * H * a.nsplits * 4);
        return;
    }
    if (esz == 4) {
        rd(a.B, b * L * G * N * 4);
        rd(a.C, b * L * G * N * 4);
    }
    rd(a.init_states, a.init_states ? b * H * P * N * 4 : 0);
    if (a.nsplits > 1) rd(a.ws_states, b * H * a.nsplits * P * N * 4);
    rd(a.z, a.z ? b * L * H * P * esz : 0);
    wr(a.y, b * L * H * P * esz);
    wr(a.final_states, a.final_states ? b * H * P * N * 4 : 0);
    const int Q = a.chunk;
    wr(a.dbg_seg, a.dbg_seg ? b * H * a.nchunks * (size_t)(4 * Q + 2 * (Q / 16) + Q / 32) * 4 : 0);
}

}  // namespace

namespace ssd {

size_t cb_s_elems(int Q) { return nblk(Q) * 64 * 8; }

// The allocation-free entry point's fixed workspace, as a host object of the
// documented size (ssd_noalloc.hip holds the device array).
void *noalloc_scratch(int, std::string *) {
    static unsigned char host_scratch[SSD_NOALLOC_WORKSPACE_BYTES];
    return host_scratch;
}

bool launch_cb(int Q, int N, const CbArgs &cb, hipStream_t) {
    ++g_launches;
    const size_t b = cb.batch, L = cb.seqlen, G = cb.ngroups;
    rd(cb.B, b * L * G * N * 2);
    rd(cb.C, b * L * G * N * 2);
    ChunkArgs a;
    memset(&a, 0, sizeof(a));
    a.ws_S = cb.ws_S;
    a.ws_BT = cb.ws_BT;
    a.ws_C = cb.ws_C;
    a.batch = cb.batch;
    a.ngroups = cb.ngroups;
    a.nchunks = cb.nchunks;
    a.chunk = Q;
    a.dstate = N;
    group_operands(a, true);
    return true;
}

bool launch_scan_bf16_q64(int, int, const ChunkArgs &a, hipStream_t) { chunk_pass(a, 2); return true; }
bool launch_scan_bf16_q128(int, int, const ChunkArgs &a, hipStream_t) { chunk_pass(a, 2); return true; }
bool launch_scan_bf16_q256(int, int, const ChunkArgs &a, hipStream_t) { chunk_pass(a, 2); return true; }
bool launch_scan_bf16_direct(int, int, const ChunkArgs &a, hipStream_t) {
    if (a.mode != kModeFull) return false;
    chunk_pass(a, 2);
    return true;
}
bool launch_scan_bf16_diff(int, int, const ChunkArgs &a, hipStream_t) {
    if (a.mode != kModeFull) return false;
    chunk_pass(a, 2);
    return true;
}
void launch_chunk_f32(int, const ChunkArgs &a, hipStream_t) { chunk_pass(a, 4); }

void launch_split_scan(const float *init_states, float *ws_states, const float *ws_decay, int batch,
                       int nheads, int nsplits, int pn, hipStream_t) {
    ++g_launches;
    const size_t bh = (size_t)batch * nheads;
    rd(init_states, init_states ? bh * pn * 4 : 0);
    rd(ws_decay, bh * nsplits * 4);
    rd(ws_states, bh * nsplits * pn * 4);
    wr(ws_states, bh * nsplits * pn * 4);
}

void launch_mask(int Q, const MaskArgs &m, hipStream_t) {
    ++g_launches;
    const size_t b = m.batch, L = m.seqlen, H = m.nheads;
    rd(m.dt, b * L * H * 4);
    rd(m.A, H * 4);
    rd(m.seq_idx, m.seq_idx ? b * L * 4 : 0);
    wr(m.out, m.out ? b * H * m.count * (size_t)Q * Q * 4 : 0);
    wr(m.sums, m.sums ? b * H * m.count * 4 : 0);
    wr(m.factors, m.factors ? b * H * m.count * (size_t)(4 * Q + 2 * (Q / 16) + Q / 32) * 4 : 0);
}

bool launch_decode(bool bf16_io, int N, const DecodeArgs &a, hipStream_t) {
    ++g_launches;
    const size_t esz = bf16_io ? 2 : 4, b = a.batch, H = a.nheads, P = a.headdim, G = a.ngroups;
    rd(a.x, b * H * P * esz);
    rd(a.dt, b * H * 4);
    rd(a.A, H * 4);
    rd(a.B, b * G * N * esz);
    rd(a.C, b * G * N * esz);
    rd(a.D, a.D ? H * 4 : 0);
    rd(a.dt_bias, a.dt_bias ? H * 4 : 0);
    rd(a.z, a.z ? b * H * P * esz : 0);
    rd(a.state, b * H * P * N * 4);
    wr(a.state, b * H * P * N * 4);
    wr(a.y, b * H * P * esz);
    return true;
}

void launch_bwd_states(bool bf16_io, const BwdArgs &a, float *out, hipStream_t) {
    ++g_launches;
    const size_t esz = bf16_io ? 2 : 4, b = a.batch, L = a.seqlen, H = a.nheads, P = a.headdim,
                 N = a.dstate, G = a.ngroups;
    // the chunks before the last (the last is never staged)
    const size_t Ls = (size_t)(a.nchunks - 1) * kBwdQ;
    for (size_t r = 0; r < b; ++r) {
        rd((const char *)a.x + r * L * H * P * esz, Ls * H * P * esz);
        rd((const char *)a.B + r * L * G * N * esz, Ls * G * N * esz);
        rd(a.dt + r * L * H, Ls * H * 4);
        rd(a.seq_idx ? a.seq_idx + r * L : nullptr, a.seq_idx ? Ls * 4 : 0);
    }
    rd(a.A, H * 4);
    rd(a.init_states, a.init_states ? b * H * P * N * 4 : 0);
    wr(out, b * H * a.nchunks * P * N * 4);
    if (a.tail_units > 0) {   // the tail walks' adjoints: dy, C, dt, seq_idx, dfinal of their rows
        rd(a.dy, b * L * H * P * esz);
        rd(a.C, b * L * G * N * esz);
        rd(a.dt, b * L * H * 4);
        rd(a.seq_idx, a.seq_idx ? b * L * 4 : 0);
        rd(a.dfinal, a.dfinal ? b * H * P * N * 4 : 0);
        wr(a.g_tail, (size_t)a.tail_units * P * N * 4);
    }
}

void launch_bwd(bool bf16_io, const BwdArgs &a, hipStream_t) {
    ++g_launches;
    const size_t esz = bf16_io ? 2 : 4, b = a.batch, L = a.seqlen, H = a.nheads, P = a.headdim,
                 N = a.dstate, G = a.ngroups;
    rd(a.x, b * L * H * P * esz);
    rd(a.dy, b * L * H * P * esz);
    rd(a.B, b * L * G * N * esz);
    rd(a.C, b * L * G * N * esz);
    rd(a.dt, b * L * H * 4);
    rd(a.A, H * 4);
    rd(a.D, a.D ? H * 4 : 0);
    rd(a.seq_idx, a.seq_idx ? b * L * 4 : 0);
    rd(a.states, a.states ? b * H * a.nchunks * P * N * 4 : 0);
    rd(a.init_states, a.init_states ? b * H * P * N * 4 : 0);
    rd(a.dfinal, a.dfinal ? b * H * P * N * 4 : 0);
    wr(a.dx, b * L * H * P * 4);
    wr(a.ddt, b * L * H * 4);
    wr(a.dB_head, b * L * H * N * 4);
    wr(a.dC_head, b * L * H * N * 4);
    rd(a.g_tail, a.tail_units > 0 ? (size_t)a.tail_units * P * N * 4 : 0);
    wr(a.dA_part, b * H * 2 * 4);
    wr(a.dD_part, b * H * 2 * 4);
    wr(a.dB, b * L * G * N * 4);
    wr(a.dC, b * L * G * N * 4);
    wr(a.dA, H * 4);
    wr(a.dD, a.dD ? H * 4 : 0);
    wr(a.dinit, a.dinit ? b * H * P * N * 4 : 0);
}

void launch_exp2_probe(uint32_t, uint32_t, uint32_t, uint32_t *out, uint32_t nthreads, hipStream_t) {
    ++g_launches;
    wr(out, (size_t)3 * nthreads * 4);
}

}  // namespace ssd

extern "C" uint64_t stub_launches(void) { return g_launches; }

// The HIP runtime queries of the planner, answered as for a device 0 that
// reports no attributes (the planner then plans for 256 compute units); the
// sanitizer build links no device runtime.
extern "C" {
hipError_t hipGetDevice(int *dev) {
    if (dev) *dev = 0;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t *dev) {
    if (dev) *dev = -1;
    return hipErrorNoDevice;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
    if (v) *v = 0;
    return hipErrorNoDevice;
}
hipError_t hipGetLastError(void) { return hipSuccess; }

const char *hipGetErrorString(hipError_t) { return "stub"; }
}
