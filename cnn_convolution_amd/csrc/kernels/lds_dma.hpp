// Device helpers shared by the matrix-core kernels that copy tiles from
// memory straight into LDS (global_load_lds_dwordx4, gfx950) and multiply
// them with v_mfma_f32_16x16x32_{f16,bf16}.
//
// A copy is one wave instruction: lane l writes its 16 bytes at LDS byte
// address base + 16*l (base in M0, wave-uniform). The copies are inline
// assembly so that the compiler adds no wait of its own before later LDS
// reads (its alias tracking of such copies is conservative across a stage
// loop and would drain every copy in flight); the kernels order them with
// explicit vector-memory waits and stage_barrier(). The compiler uses M0 for
// nothing else in these kernels (their assembly has no other M0 access).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace im2win {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// D += A * B for one 16x16 output block and 32 K values: lane l holds A row
// l%16 and B column l%16, K values 8*(l/16) .. 8*(l/16)+7 of each.
template <bool BF16>
__device__ __forceinline__ floatx4_t mfma16x16x32(const uint4 &a, const uint4 &b, const floatx4_t &c)
{
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    }
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier between K stages: this wave's LDS accesses are complete
// (lgkmcnt(0)) before it signals, so no wave overwrites a buffer another wave
// may still be reading; the compiler may move no LDS access across it. It is
// the raw s_barrier: a workgroup memory fence would also make every wave
// wait for all of its copies in flight.
__device__ __forceinline__ void stage_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One wave copy of 16 bytes per lane from global memory into the LDS block at
// byte address lds (wave-uniform).
__device__ __forceinline__ void copy_to_lds(const void *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}

typedef const __attribute__((address_space(3))) uint16_t *lds_u16_ptr;

// LDS byte offset of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const uint16_t *p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16_ptr)p));
}

constexpr int kStageK = 64;   // halves per stage row: 128 bytes, 8 granules of 16 bytes

}  // namespace im2win
