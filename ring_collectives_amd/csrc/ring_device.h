// ring_device.h -- device helpers shared by the ring kernels and the fused
// GEMM + reduce-scatter kernel: tile-bounded memory access with explicit
// cache scope, and the per-tile flag protocol.
#pragma once

#include <hip/hip_runtime.h>

#include "ring_internal.h"

namespace ringc {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- memory access
// Every access goes through a buffer descriptor over exactly one tile, so the
// hardware drops any store and zeroes any load that falls outside it (the
// ragged last tile of a chunk needs no separate path).
//
// Cache policy (CDNA3/4 scope bits on the instruction itself):
//   DEV  (sc1) device scope: a store is written through to the device's
//        coherence point and a load does not return a stale copy from this
//        CU's L1 or this XCD's L2.  Used for every access that crosses ranks
//        (what a rank stores for its neighbour, what it loads from it).
//   PLAIN      default caching: a rank's own input, and results no other wave
//        reads before the launch ends.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (unformatted) 32-bit buffer
enum { POL_PLAIN = 0, POL_NT = 2, POL_DEV = 16 };

__device__ __forceinline__ rsrc_t tile_view(const void* base, long long bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}
template <int POL> __device__ __forceinline__ u32x4 ld16(rsrc_t v, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b128(v, off, 0, POL);
}
template <int POL> __device__ __forceinline__ void st16(u32x4 x, rsrc_t v, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b128(x, v, off, 0, POL);
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <int POL> __device__ __forceinline__ u32x2 ld8(rsrc_t v, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b64(v, off, 0, POL);
}
template <int POL> __device__ __forceinline__ void st8(u32x2 x, rsrc_t v, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b64(x, v, off, 0, POL);
}
template <int POL> __device__ __forceinline__ unsigned ld4(rsrc_t v, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b32(v, off, 0, POL);
}
template <int POL> __device__ __forceinline__ void st4(unsigned x, rsrc_t v, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b32(x, v, off, 0, POL);
}
// Load with a wave-uniform byte offset `soff` (kept in a scalar register).
//
// There is deliberately no store of that form.  The compiler inserts no wait
// states between a buffer store of more than 8 bytes whose offset sits in a
// scalar register and a following VALU write of the store's data registers,
// and on gfx950 such a write, issued right after a 16-byte store, reached
// memory in place of the stored value for part of the wave (seen with two
// waves per SIMD).  Stores therefore carry their whole offset in the vector
// register (soffset 0), the form the compiler does protect.
template <int POL> __device__ __forceinline__ u32x4 ld16s(rsrc_t v, unsigned voff, unsigned soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(v, voff, soff, POL);
}
template <int POL> __device__ __forceinline__ unsigned short ld2(rsrc_t v, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b16(v, off, 0, POL);
}
template <int POL> __device__ __forceinline__ void st2(unsigned short x, rsrc_t v, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b16(x, v, off, 0, POL);
}

// ---------------------------------------------------------------- flags
// A flag is one int in HBM, kFlagStride ints apart from the next.  It goes
// from 0 to 1 when its producer has finished a tile, and back to 0 when its
// single consumer has seen it (so a finished launch leaves the table zeroed).

// Record the first asynchronous error of a launch and where it happened
// (later errors keep the first one).
__device__ inline void report_error(Status* st, int code, int r, int k, int j) {
    int expected = 0;
    if (__hip_atomic_compare_exchange_strong(&st->code, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
        int info = (r & 0xFF) | ((k & 0xFF) << 8) | ((j < 32767 ? j : 32767) << 16);
        __hip_atomic_store(&st->info, info, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}
__device__ inline void report_timeout(Status* st, int r, int k, int j) { report_error(st, RING_ETIMEOUT, r, k, j); }

// ---------------------------------------------------------------- workspace record
// A launch reads the record of data earlier calls left in the workspace
// (Status::data_lo_inv, data_hi) as it starts; the loads are issued at once
// and their result is needed only by ws_ok, by when the wave's first data
// loads have usually returned too.
struct WsRecord {
    unsigned long long lo_inv, hi;
};
__device__ __forceinline__ WsRecord ws_record(Status* st) {
    WsRecord r;
    r.lo_inv = __hip_atomic_load(&st->data_lo_inv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    r.hi = __hip_atomic_load(&st->data_hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return r;
}
// The launch's own data span joins the record (one lane of one wave per
// launch).  The record only grows, to the smallest range holding every span
// added since the last zero fill.  Every span lies past the status block;
// the span a launch checks (its flags or words and everything below them)
// starts right at the end of the status block, and its own data lies above
// it.  So a record that clears the checked span lies wholly above it, and
// still does once the launch's own data has joined: every wave of a launch
// gets the same answer, whether it reads the record before or after the
// launch's own addition.
__device__ __forceinline__ void ws_add_data(Status* st, WsSpan data) {
    if (data.hi > data.lo) {
        __hip_atomic_fetch_max(&st->data_lo_inv, ~data.lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_max(&st->data_hi, data.hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}
// False if data an earlier call left may lie where this launch needs zeros
// (its flags or words): RING_EWORKSPACE is recorded and the wave must stop
// before it signals anything.
__device__ __forceinline__ bool ws_ok(Status* st, const WsRecord& rec, WsSpan zero, int lane) {
    const unsigned long long lo = ~rec.lo_inv;
    if (lo < zero.hi && zero.lo < rec.hi) {
        if (lane == 0) report_error(st, RING_EWORKSPACE, 0, 0, 0);
        return false;
    }
    return true;
}

// First look at a flag; callers issue their independent loads before they
// spin on the result.
__device__ __forceinline__ int peek_flag(const int* f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin until flag f is set (unless `seen` already is), then clear it (unless
// `clear` is false: a flag with several readers is cleared by the kernel
// that owns it once every reader is done).
// Returns false if the launch is being abandoned (this wave timed out, or
// another one did).  The loads of the neighbour's data that follow are
// device-scope and are issued only after the flag was seen (control
// dependency; the empty asm keeps the compiler from hoisting them).
// (r, k, j) only label a timeout report.
__device__ inline bool wait_flag(int* f, Status* st, long long spin_limit, int r, int k, int j,
                                 int lane, int seen, bool clear = true) {
    if (seen < 1) {
        const long long t0 = wall_clock64();
        unsigned spins = 0;
        while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < 1) {
            __builtin_amdgcn_s_sleep(2);
            if ((++spins & 31u) == 0) {
                if (__hip_atomic_load(&st->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
                    return false;
                if (wall_clock64() - t0 > spin_limit) {
                    if (lane == 0) report_timeout(st, r, k, j);
                    return false;
                }
            }
        }
    }
    asm volatile("" ::: "memory");
    // This wave is the flag's only reader in this launch: clear it for the next.
    if (clear && lane == 0) __hip_atomic_store(f, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Publish: wait until all of this wave's memory operations are complete (its
// device-scope stores are at the coherence point, its loads of the
// neighbour's data have returned), then set flag f.  With `check` (a debug
// knob) the add returns the flag's old value, which must be 0: each flag is
// set exactly once per launch and cleared by its reader, so anything else
// means two producers or a missed clear, recorded as RING_EPROTOCOL at
// (r, k, j).
__device__ __forceinline__ void signal_flag(int* f, int lane, int check, Status* st, int r, int k, int j) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) {
        if (check) {
            const int old = __hip_atomic_fetch_add(f, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old != 0) report_error(st, RING_EPROTOCOL, r, k, j);
        } else {
            __hip_atomic_fetch_add(f, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace ringc
