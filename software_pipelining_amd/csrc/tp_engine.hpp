// Device-side building blocks of the global->LDS copy pipeline (gfx950 only).
//
// The pages build their pipelines from an asynchronous copy that returns at
// once, a per-thread "wait until at most N of my copy groups are pending", and
// a block barrier ("Asynchronous Copies", section "A Global-to-Shared Copy":
// commit_group / wait_group / cta_sync; "Asynchronous Data Movement", section
// "Barriers and pipelines": producer_commit / consumer_wait /
// consumer_release). On CDNA4 those map onto:
//
//   asynchronous copy  -> buffer_load_{dword,dwordx4,ubyte} ... lds: the data
//                         goes from memory straight into LDS at
//                         M0 + lane * width, never through VGPRs;
//   wait_group(N)      -> s_waitcnt vmcnt(N): a wave's vector-memory
//                         operations retire in issue order, so "at most N
//                         outstanding" means everything issued before the last
//                         N has landed;
//   cta_sync           -> s_barrier, after the wait, so every wave of the
//                         workgroup sees every lane's LDS data.
//
// Every memory instruction here is inline assembly. The compiler therefore
// never sees an LDS-DMA write (it would otherwise wait for all of them,
// vmcnt(0), before every LDS read and serialize the pipeline), and the number
// of memory instructions a wave issues is exactly what the wait counts assume.
// Predication uses the buffer resource's range check instead of branches: a
// lane whose offset is not below num_records moves no data (a load into LDS
// writes zeros there, a store is dropped), yet the instruction still issues,
// so counts never depend on data. Out-of-range offsets used here stay small:
// at most a few tiles past num_records, never near 2^31.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {
namespace dev {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource descriptor (V#) of a raw byte-addressed buffer: 48-bit base,
// stride 0 (unstructured, range-checked against num_records in bytes), data
// format 32-bit (word 3 = 0x00020000 on gfx9-family parts), no swizzle.
struct BufferRes {
    u32x4 d;
};

__device__ __forceinline__ BufferRes make_buffer_res(const void *base, uint32_t num_records)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    BufferRes r;
    r.d.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.d.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    r.d.z = __builtin_amdgcn_readfirstlane(num_records);
    r.d.w = 0x00020000u;
    return r;
}

// Byte address of a generic pointer into LDS, as the 32-bit LDS offset that
// M0 and ds_* instructions take.
__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// The descriptor operand of a buffer instruction must live in SGPRs; this
// keeps it there even if register allocation moved the value to VGPRs.
__device__ __forceinline__ u32x4 sgpr_res(const BufferRes &r)
{
    return u32x4{uniform(r.d.x), uniform(r.d.y), uniform(r.d.z), uniform(r.d.w)};
}

// Lambdas that carry a kernel's per-tile steps are always inlined, so their
// captures stay in registers.
#define TP_INLINE __attribute__((always_inline))

// ------------------------------------------------------ hazards (wait states)
// The compiler's hazard recognizer cannot see inside inline assembly, so every
// asm block below carries the wait states its buffer instruction needs:
//   - a VALU write of an SGPR (e.g. the v_readfirstlane that rebuilds a
//     descriptor the compiler kept in VGPRs) followed by a vector-memory
//     instruction reading that SGPR needs 5 wait states: "s_nop 4" right
//     before every buffer instruction;
//   - an SALU write of M0 followed by an LDS-DMA load needs 1: the same nop;
//   - a store of more than 8 bytes followed by a VALU write of its data VGPRs
//     needs 2 on this architecture family (the store reads its data late):
//     "s_nop 1" right after every 16-byte store. With one wait state the
//     compiler's next instruction may overwrite the first data register
//     before the store has read it, and that dword of the chunk is stored
//     wrong, now and then.

// Cache-policy modifiers of the streaming loads and stores (compile-time).
// Streamed data is touched once: loads are non-temporal, stores are
// non-temporal at device scope (written through to memory rather than kept
// dirty in the XCD's L2). Measured on the 2^28-float map: non-temporal LDS-DMA
// loads move ~10 % more bytes per second than default-policy loads, and
// device-scope stores a further 1-5 %.
#ifndef TP_LOAD_CPOL
#define TP_LOAD_CPOL " nt"
#endif
#ifndef TP_STORE_CPOL
#define TP_STORE_CPOL " sc1 nt"
#endif

// ------------------------------------------------------- async copies to LDS
// Lane l's bytes land at LDS address m0 + l * width (m0 wave-uniform).
// `voff` is the lane's byte offset inside the resource. M0 is written without
// being declared: the compiler reserves it and rejects it as a clobber. The
// built kernels use M0 nowhere else (tests/test_isa_hazards.py checks that
// every mention of M0 is one of these writes, followed by its load).
__device__ __forceinline__ void dma_b128(const BufferRes &r, uint32_t voff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 4\n\t"
                 "buffer_load_dwordx4 %0, %1, 0 offen" TP_LOAD_CPOL " lds"
                 :
                 : "v"(voff), "s"(sgpr_res(r)), "s"(m0)
                 : "memory");
}

__device__ __forceinline__ void dma_b32(const BufferRes &r, uint32_t voff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 4\n\t"
                 "buffer_load_dword %0, %1, 0 offen" TP_LOAD_CPOL " lds"
                 :
                 : "v"(voff), "s"(sgpr_res(r)), "s"(m0)
                 : "memory");
}

// One byte per lane; lane l's byte lands in the low byte of the dword at
// m0 + 4 * l (LDS-DMA writes a dword slot per lane for sub-dword loads).
__device__ __forceinline__ void dma_u8(const BufferRes &r, uint32_t voff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 4\n\t"
                 "buffer_load_ubyte %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(sgpr_res(r)), "s"(m0)
                 : "memory");
}

// ----------------------------------------------------------------- stores
// Streaming stores: the results are not read again by this kernel.
__device__ __forceinline__ void store_b128(const BufferRes &r, uint32_t voff, u32x4 v)
{
    asm volatile("s_nop 4\n\t"
                 "buffer_store_dwordx4 %0, %1, %2, 0 offen" TP_STORE_CPOL "\n\t"
                 "s_nop 1"
                 :
                 : "v"(v), "v"(voff), "s"(sgpr_res(r))
                 : "memory");
}

__device__ __forceinline__ void store_b32(const BufferRes &r, uint32_t voff, uint32_t v)
{
    asm volatile("s_nop 4\n\t"
                 "buffer_store_dword %0, %1, %2, 0 offen" TP_STORE_CPOL
                 :
                 : "v"(v), "v"(voff), "s"(sgpr_res(r))
                 : "memory");
}

// ------------------------------------------- hand-offs between workgroups
// A workgroup that hands data to another, possibly on another XCD, reads and
// writes it at device scope (sc1); the L2s of the XCDs are not coherent with
// one another. Device-scope loads and stores are what the compiler itself
// emits for relaxed atomic loads and stores at device ("agent") scope on
// gfx950, with no L2 write-back or invalidate: they are coherent across XCDs
// on their own. The compiler implements relaxed 64-bit atomics the same way,
// with one 8-byte access (dwordx2): an aligned 8-byte device-scope store
// becomes visible as a whole. So a 4-byte data word stored together with a
// 4-byte tag in one such access needs no flag and no fence: a receiver whose
// 8-byte load finds the tag has the data that came with it. (The compiler's
// release and acquire sequences would add an L2 write-back (buffer_wbl2) and
// invalidate (buffer_inv) that act on the whole L2 of an XCD; a flag protocol
// built on them took 19 ms for 2^20 hand-offs.)

// A 4-byte load at device scope into a register, complete when this returns
// (the wait is part of the block, so the compiler sees the value only then).
__device__ __forceinline__ uint32_t load_b32_device(const BufferRes &r, uint32_t voff)
{
    uint32_t v;
    asm volatile("s_nop 4\n\t"
                 "buffer_load_dword %0, %1, %2, 0 offen sc1\n\t"
                 "s_waitcnt vmcnt(0)"
                 : "=v"(v)
                 : "v"(voff), "s"(sgpr_res(r))
                 : "memory");
    return v;
}

// An 8-byte load at device scope, one access, complete when this returns.
__device__ __forceinline__ uint64_t load_b64_device(const BufferRes &r, uint32_t voff)
{
    uint64_t v;
    asm volatile("s_nop 4\n\t"
                 "buffer_load_dwordx2 %0, %1, %2, 0 offen sc1\n\t"
                 "s_waitcnt vmcnt(0)"
                 : "=v"(v)
                 : "v"(voff), "s"(sgpr_res(r))
                 : "memory");
    return v;
}

// A 4-byte store at device scope (a header or status word).
__device__ __forceinline__ void store_b32_device(const BufferRes &r, uint32_t voff, uint32_t v)
{
    asm volatile("s_nop 4\n\t"
                 "buffer_store_dword %0, %1, %2, 0 offen sc1"
                 :
                 : "v"(v), "v"(voff), "s"(sgpr_res(r))
                 : "memory");
}

// An 8-byte store at device scope, one access (a tagged word).
__device__ __forceinline__ void store_b64_device(const BufferRes &r, uint32_t voff, uint64_t v)
{
    asm volatile("s_nop 4\n\t"
                 "buffer_store_dwordx2 %0, %1, %2, 0 offen sc1"
                 :
                 : "v"(v), "v"(voff), "s"(sgpr_res(r))
                 : "memory");
}

// ------------------------------------------------------------ completion
// Wait until at most K of this wave's vector-memory operations are pending.
template <int K>
__device__ __forceinline__ void vm_wait()
{
    static_assert(K >= 0 && K <= 63, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(K) : "memory");
}

// Workgroup barrier; also a compiler barrier so no LDS access moves across it.
__device__ __forceinline__ void block_sync()
{
    asm volatile("s_barrier" : : : "memory");
}

// ------------------------------------------------------------- the engine
// What a kernel body is written against: the workgroup's indices, its LDS,
// and the primitives above. Each kernel here is a thin __global__ wrapper
// that instantiates its body (a template on the engine type) with this
// engine. The same bodies compile on the host against the CPU emulator in
// tests/emu, which runs every wave in lock-step and checks each access
// against the caller's buffers, each LDS read against the waits that must
// have retired its load, and LDS shared between waves against the barriers.
struct GpuEngine {
    uint8_t *lds;        // the workgroup's dynamic LDS
    uint32_t nthreads_;  // blockDim.x, read in the kernel itself (see gpu_engine)

    __device__ __forceinline__ uint32_t tid() const { return threadIdx.x; }
    __device__ __forceinline__ uint32_t nthreads() const { return nthreads_; }
    __device__ __forceinline__ uint32_t block() const { return blockIdx.x; }
    __device__ __forceinline__ uint32_t blocks() const { return gridDim.x; }
    __device__ __forceinline__ uint32_t uniform(uint32_t v) const { return dev::uniform(v); }
    // LDS address of lds[0], as M0 takes it
    __device__ __forceinline__ uint32_t lds_base() const { return lds_offset(lds); }
    template <class T>
    __device__ __forceinline__ T lds_load(uint32_t off) const
    {
        return *reinterpret_cast<const T *>(lds + off);
    }
    // A wave's own write into LDS (ds_write). LDS operations of one wave
    // execute in order, so the wave's later reads of these bytes see them.
    template <class T>
    __device__ __forceinline__ void lds_store(uint32_t off, T v) const
    {
        *reinterpret_cast<T *>(lds + off) = v;
    }
    __device__ __forceinline__ BufferRes res(const void *base, uint32_t num_records) const
    {
        return make_buffer_res(base, num_records);
    }
    __device__ __forceinline__ void dma_b128(const BufferRes &r, uint32_t voff, uint32_t m0) const
    {
        dev::dma_b128(r, voff, m0);
    }
    __device__ __forceinline__ void dma_b32(const BufferRes &r, uint32_t voff, uint32_t m0) const
    {
        dev::dma_b32(r, voff, m0);
    }
    __device__ __forceinline__ void dma_u8(const BufferRes &r, uint32_t voff, uint32_t m0) const
    {
        dev::dma_u8(r, voff, m0);
    }
    __device__ __forceinline__ void store_b128(const BufferRes &r, uint32_t voff, u32x4 v) const
    {
        dev::store_b128(r, voff, v);
    }
    __device__ __forceinline__ void store_b32(const BufferRes &r, uint32_t voff, uint32_t v) const
    {
        dev::store_b32(r, voff, v);
    }
    template <int K>
    __device__ __forceinline__ void wait() const
    {
        vm_wait<K>();
    }
    __device__ __forceinline__ void barrier() const { block_sync(); }
    __device__ __forceinline__ uint32_t load_b32_device(const BufferRes &r, uint32_t voff) const
    {
        return dev::load_b32_device(r, voff);
    }
    __device__ __forceinline__ uint64_t load_b64_device(const BufferRes &r, uint32_t voff) const
    {
        return dev::load_b64_device(r, voff);
    }
    __device__ __forceinline__ void store_b32_device(const BufferRes &r, uint32_t voff, uint32_t v) const
    {
        dev::store_b32_device(r, voff, v);
    }
    __device__ __forceinline__ void store_b64_device(const BufferRes &r, uint32_t voff, uint64_t v) const
    {
        dev::store_b64_device(r, voff, v);
    }
    // true on every lane when p holds on every lane of the wave (a ballot)
    __device__ __forceinline__ bool all_lanes(bool p) const
    {
        return __builtin_amdgcn_ballot_w64(!p) == 0;
    }
    // a short pause between polls
    __device__ __forceinline__ void pause() const { __builtin_amdgcn_s_sleep(1); }
};

// The engine of a kernel whose dynamic LDS is `lds`. blockDim.x is read here,
// in the kernel's own body: read inside the inlined kernel body instead, the
// compiler no longer folds it to the launch's uniform group size and loads
// the group size from the implicit arguments with a vector load.
#define TP_GPU_ENGINE(lds) (::tp::dev::GpuEngine{(lds), blockDim.x})

// ---------------------------------------------------------------- helpers
template <int Begin, int End, typename F>
__host__ __device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (Begin < End) {
        f(std::integral_constant<int, Begin>{});
        static_for<Begin + 1, End>(static_cast<F &&>(f));
    }
}

}  // namespace dev
}  // namespace tp
