// LDS staging helpers shared by the gfx950 prefill kernels (forward and backward): the XOR swizzle of
// 256-byte LDS rows, transposed LDS reads, buffer loads that write LDS directly, explicit waits and
// barriers, and instruction-scheduling fences.  wave64 only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufWord3 = 0x00020000; // raw buffer resource word 3 (gfx9 family)

// XOR swizzle of the 16 chunk slots (16 B each) of a 256-B LDS row: chunk c of row r sits in slot
// c ^ swz(r % 16).  It keeps 16-B reads along a column of rows and the transposed 8-B reads of
// ds_read_b64_tr_b16 free of bank conflicts.
__device__ __forceinline__ int swz(int r)
{
    return ((r & 1) ? 10 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0);
}

// s_waitcnt immediates (gfx9 layout: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier without a memory-model fence: the caller has already waited for what it needs.
__device__ __forceinline__ void barrier()
{
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// Waits until at most N of this wave's vector memory loads are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(wait_vm(N));
    compiler_fence();
}

// Keeps a computed value at this point of the instruction stream (the compiler would otherwise sink it
// to its first use and undo a hand-made interleaving).
__device__ __forceinline__ void anchor(uint32_t v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void anchor(float v) { asm volatile("" ::"v"(v)); }
// No instruction may be scheduled across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ds_read_b64_tr_b16: in each 16-lane group, lane j addresses 4 bf16 of row k0 + j/4, columns
// c0 + 4 (j%4) .. +3 of a 4 x 16 block; lane i receives column c0 + i of rows k0 .. k0+3.
__device__ __forceinline__ uint2 lds_read_tr(const char *p)
{
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(uint2, r);
}

// Raw buffer resource: base address, no stride, num_records bytes.  A load whose offset (per-lane VGPR
// offset plus scalar offset plus instruction offset) reaches past num_records returns zero on gfx950.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_records)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)num_records, kBufWord3};
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void *)(p));
}

// Buffer loads written straight to LDS: lane l's 16 (dma16) or 4 (dma4) bytes land at lds + 16 l (or
// 4 l).  Written as inline asm so that the compiler does not fold them into its own wait bookkeeping
// (which cannot tell LDS stages apart and would drain every load in flight before each LDS read); they
// return no registers, and every wait for them is explicit (wait_vmcnt).
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rsrc, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}
// dma16 to lds + OFF: the offset is added while m0 is set (an immediate), so a caller issuing several
// chunks from one base keeps one scalar register for them instead of one per chunk.
template <uint32_t OFF>
__device__ __forceinline__ void dma16_at(uint32_t lds, uint32_t voff, i32x4 rsrc, uint32_t soff)
{
    asm volatile("s_add_u32 m0, %0, %4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF)
                 : "memory", "scc");
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, i32x4 rsrc, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}

} // namespace attn
