// ring.hpp -- compile-time helpers of the weight-streaming kernels
// (internal): loops with compile-time indices and explicit waits for vector
// memory loads.
#pragma once

#include <type_traits>

#include "kstep.hpp"

namespace lmhead {

// Calls f(std::integral_constant<int, 0>{}) ... f(integral_constant<N - 1>)
// in order: loops whose index must be a compile-time constant.
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

// Waits until at most N of this wave's vector memory loads are outstanding.
// Loads complete in issue order, so this retires every load but the last N
// issued. Fenced, so the compiler moves no instruction across it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  constexpr int ENC = (N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00;  // vmcnt(N) only
  sched_fence();
  __builtin_amdgcn_s_waitcnt(ENC);
  sched_fence();
}

// Waits until this wave's LDS operations have completed (lgkmcnt(0)): before
// a direct-to-LDS load overwrites LDS this wave has just read, since such a
// load writes LDS on its own path, not behind the wave's earlier ds_reads.
__device__ __forceinline__ void wait_lds() {
  sched_fence();
  __builtin_amdgcn_s_waitcnt(0xC07F);
}

// The issue schedule of a wave that streams its weight through a ring of NSL
// LDS slots, in units: unit u is (chunk u / NB, column block u % NB). Its LPU
// direct loads are issued when unit u - NSL has been read (units 0 .. NSL - 1
// in the prologue), into slot u % NSL; right after the loads of a chunk's
// first unit come the HL hidden loads of that chunk, into register set
// (chunk % NHR). Vector memory loads complete in issue order, so each wait is
// "all but the loads issued after X".
template <int NB, int NSL, int HL, int LPU>
struct Schedule {
  static constexpr int hid(int w) { return ((w % NB) + NB) % NB == 0 ? HL : 0; }
  // before the first read of unit u: loads issued after unit u's
  static constexpr int wait_unit(int u) {
    int n = hid(u);
    for (int w = u + 1; w <= u + NSL - 1; ++w) n += LPU + hid(w);
    return n;
  }
  // at the end of the chunk whose last unit is u, after unit u + NSL was
  // issued: loads issued after the next chunk's hidden loads (which follow
  // unit u + 1's)
  static constexpr int wait_hidden(int u) {
    int n = 0;
    for (int w = u + 2; w <= u + NSL; ++w) n += LPU + hid(w);
    return n;
  }
  // hidden chunks held in registers at once: chunk c is issued with unit
  // c NB - NSL and written to LDS at the end of chunk c - 1
  static constexpr int NHR = (NSL - 1) / NB + 1;
  // units per unrolled period: slots, register sets and the two LDS hidden
  // buffers all at compile-time positions
  static constexpr int PERIOD = lcm_c(lcm_c(NB * NHR, NSL), 2 * NB);
};

// The NVFP4 ring kernel's issue schedule (nvfp4.hip): units of 256-element
// chunks with two direct loads each, the hidden loads of a chunk after its
// first unit's, and each block's scales loaded for a group of eight chunks
// at once.
constexpr int pow2_at_least(int n, int p = 1) { return p >= n ? p : pow2_at_least(n, 2 * p); }

template <int NB, int NSL, int HL>
struct NvSchedule {
  static constexpr int GROUP = 8;  // chunks per scale group
  static constexpr int md(int a, int m) { return ((a % m) + m) % m; }
  static constexpr int chunk8(int v) { return md(v >= 0 ? v / NB : -((-v + NB - 1) / NB), GROUP); }
  static constexpr int hid(int w) { return md(w, NB) == 0 ? HL : 0; }
  static constexpr int scl(int v) { return chunk8(v) == GROUP - 1 ? 2 : 0; }
  static constexpr int batch(int v) { return 2 + hid(v + NSL) + scl(v); }
  // before the first read of unit u: loads after unit u's two direct loads
  static constexpr int wait_unit(int u) {
    int n = hid(u) + scl(u - NSL);
    for (int v = u - NSL + 1; v <= u - 1; ++v) n += batch(v);
    return n;
  }
  // before the first read of a scale group at unit u (the group's first
  // chunk): the group was loaded last in batch u - NB
  static constexpr int wait_scale(int u) {
    int n = 0;
    for (int v = u - NB + 1; v <= u - 1; ++v) n += batch(v);
    return n;
  }
  static constexpr int wait_first(int u) {
    return chunk8(u) == 0 && wait_scale(u) < wait_unit(u) ? wait_scale(u) : wait_unit(u);
  }
  // hidden chunks held in registers at once: chunk c is issued in batch
  // c NB - NSL and stored at the end of unit c NB - 1 (rounded up to a power
  // of two, which keeps the period short)
  static constexpr int NHR = pow2_at_least((NSL - 1) / NB + 1);
  // units per unrolled period: slots, register sets, scale groups and the two
  // LDS hidden buffers all at compile-time positions
  static constexpr int PERIOD = lcm_c(lcm_c(lcm_c(NB * GROUP, NSL), NB * NHR), 2 * NB);
  // at the end of the chunk whose last unit is u (after batch u): loads
  // after the next chunk's hidden loads, which sit in batch u + 1 - NSL
  static constexpr int wait_hidden(int u) {
    int n = scl(u + 1 - NSL);
    for (int v = u + 2 - NSL; v <= u; ++v) n += batch(v);
    return n;
  }
};

typedef __attribute__((address_space(3))) void lds_void_t;

// One direct-to-LDS load of 16 bytes per active lane: lane l's bytes land at
// LDS dst + 16 l (dst wave-uniform). These loads carry the weight stream,
// read once per call, so they are marked non-temporal: measured on MI355X,
// the decode head's stream went from 5.8 to 6.6 TB/s (180 -> 159 µs at
// M = 1) once it stopped displacing the caches' other contents -- the
// hidden rows every work-group reads again.
__device__ __forceinline__ void dma16_lds(rsrc_t r, void *dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, voff, soff, 0, LOAD_STREAM);
}

}  // namespace lmhead
