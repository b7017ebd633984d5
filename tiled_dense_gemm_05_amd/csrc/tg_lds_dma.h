// Device helpers shared by the kernels that stage operands straight from
// global memory into LDS (gfx950 buffer_load ... lds) and order that traffic
// themselves with counter waits and barriers.  These are the two AMD
// pipeline primitives the "TileLang paper reading" page (hotelren.com),
// section 3, names: loads that write LDS without passing through registers,
// and s_waitcnt vmcnt waits that release a stage once its loads have landed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {
namespace dma {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// A buffer offset at or past a descriptor's record count reads as zero; the
// kernels give out-of-range chunks this offset (== make_rsrc's record count).
constexpr uint32_t kOutOfRange = 0x80000000u;

// s_waitcnt vmcnt(N), other counters untouched, fenced against compiler
// reordering of memory operations.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt");
    constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(imm);
    asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS operations have completed.
__device__ __forceinline__ void wait_lgkm0()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((3 << 14) | (0 << 8) | (7 << 4) | 15);
    asm volatile("" ::: "memory");
}

// Workgroup barrier once this wave's LDS operations have completed (the
// lgkmcnt wait is a builtin so the compiler's own wait tracking sees it).
__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((3 << 14) | (0 << 8) | (7 << 4) | 15);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Raw buffer descriptor over `base` with `records` bytes (offsets at or past
// it read as zero), 32-bit data format as the gfx9 family requires.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t records = kOutOfRange)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane((int)records);
    r.w = 0x00020000;
    return r;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from rsrc + voff into the 1 KiB LDS block at lds_addr
// (lane L at byte 16 L; the block base goes through M0).
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "m0");
}

// The same with the non-temporal hint: data streamed once is not kept in the
// caches.
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "m0");
}
#pragma clang diagnostic pop

}  // namespace dma
}  // namespace tg
