// LDS tile helpers shared by the bf16 kernels: the swizzled row-major tile
// layout, workgroup barriers and asynchronous direct-to-LDS row staging.
#pragma once

#include "ssd_common.hpp"

namespace ssd {

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

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8; an all-ones field does not wait).  The waits are
// issued through the builtin rather than inline assembly so that the
// compiler's own wait placement sees them and knows what has completed.
constexpr int kWaitLgkm0 = 0xC07F;        // lgkmcnt(0)
constexpr int kWaitVmemLgkm0 = 0x0070;    // vmcnt(0) lgkmcnt(0)

// vmcnt(vm) lgkmcnt(0), vm < 64
constexpr int wait_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }
// vmcnt(vm) only, vm < 64
constexpr int wait_vm(int vm) { return wait_vm_lgkm0(vm) | (15 << 8); }

// Workgroup barrier ordering LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (the prefetch).
__device__ inline void lds_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Barrier after which every direct-to-LDS load issued before it has landed.
__device__ inline void vmem_lds_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(kWaitVmemLgkm0);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The same, except that the KEEP most recently issued vector-memory
// operations may still be in flight (completions are counted in issue order,
// so everything older has landed).  The caller issues exactly KEEP operations
// after the last one it needs, behind a compiler fence.
template <int KEEP>
__device__ inline void vmem_lds_sync_keep() {
    static_assert(KEEP >= 0 && KEEP < 64, "vmcnt range");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(KEEP));
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Barrier after which every direct-to-LDS load has landed except the KEEP
// most recently issued ones, which are themselves direct-to-LDS loads of a
// later tile that no wave reads before a later barrier (loads run ahead by
// one more tile).  The marker lets the build check verify that exactly the
// KEEP newest vector-memory operations before the wait are those loads.
template <int KEEP, int TAG>
__device__ inline void vmem_lds_sync_lookahead() {
    static_assert(KEEP > 0 && KEEP < 64, "vmcnt range");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    asm volatile("; ssd lookahead wait %0" ::"i"(TAG) : "memory");
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(KEEP));
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// An L2 prefetch: one direct-to-LDS load of a 1 KB block (64 lanes x 16
// bytes) into a scratch LDS block that nothing reads, issued only to bring
// the block's lines into L2 ahead of the load that uses them.  The marker
// tells the build check that this direct-to-LDS load may stay in flight
// across a barrier (vmem_lds_sync_touch).
__device__ inline void l2_touch(const void *src, void *lds_scratch) {
    asm volatile("; ssd touch" ::: "memory");
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)lds_scratch, 16, 0, 0);
}

// Barrier after which every vector-memory operation has completed except the
// KEEP most recently issued ones, which are stores, ordinary loads or
// l2_touch prefetches (nothing the barrier publishes).  The build check
// verifies that every direct-to-LDS load among them follows a touch marker.
template <int KEEP>
__device__ inline void vmem_lds_sync_touch() {
    static_assert(KEEP > 0 && KEEP < 64, "vmcnt range");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    asm volatile("; ssd touch wait" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(KEEP));
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 16 zero bytes in global memory: the source of the padding rows of a tile.
static __device__ __attribute__((aligned(16))) const bf16 kZeroChunk[8] = {};

// Asynchronously copy rows [0, nvalid) of a Q-row tile (CPR 16-byte chunks
// per row, row r at src + r * gstride elements) into a swizzled LDS tile, and
// zeros into rows [nvalid, Q).  Every wave issues whole 1 KB blocks: block k
// covers LDS slots [64 k, 64 k + 64), lane l fills slot 64 k + l (row
// slot / CPR, physical chunk slot % CPR) from the global chunk that the
// swizzle puts there.  Straight-line code with a fixed number of loads per
// wave, so that the compiler can count them when it places its waits.
template <int Q, int W, int CPR>
__device__ inline void stage_rows_async(bf16 *lds, const bf16 *src, int64_t gstride, int nvalid,
                                        int wave, int lane) {
    constexpr int nblk = Q * CPR / 64;
    constexpr int per = (nblk + W - 1) / W;
    static_assert(Q * CPR % 64 == 0, "whole 1 KB blocks");
#pragma unroll
    for (int kk = 0; kk < per; ++kk) {
        const int k = wave + kk * W;
        if (nblk % W != 0 && k >= nblk) break;
        const int slot = k * 64 + lane;
        const int r = slot / CPR, pc = slot % CPR;
        const int c = pc ^ swz<CPR>(r);
        const bf16 *g = (r < nvalid) ? src + (int64_t)r * gstride + c * 8 : kZeroChunk;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                         (__attribute__((address_space(3))) void *)(lds + k * 512),
                                         16, 0, 0);
    }
}

}  // namespace ssd
