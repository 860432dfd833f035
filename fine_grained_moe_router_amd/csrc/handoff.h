// handoff.h -- global-address-space access and the tagged hand-off words by which the
// workgroups of a persistent kernel (gfx950) pass data to one another.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace dev {

// Every access to device memory goes through the global address space: the pointers
// here arrive as generic pointers (from the argument block and the weight table), and
// generic (flat) accesses also count against the LDS wait counter, so an LDS wait would
// otherwise wait for weight loads and hand-off stores still in flight.
#define GAS __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ GAS T *glb(T *p) { return (GAS T *)p; }
// A 16-byte load through the global address space.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const void *p) {
    const u32x4 v = *(const GAS u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
// The same for a weight stream read once per call: the nontemporal hint (streaming MI355X
// reads measured about 10 % faster with it: 6.7 against 6.1 TB/s for a 4 GiB read).
__device__ __forceinline__ uint4 ld16nt(const void *p) {
    const u32x4 v = __builtin_nontemporal_load((const GAS u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld8(const void *p) {
    const u32x2 v = *(const GAS u32x2 *)p;
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st32(void *p, uint32_t v) {
    __hip_atomic_store(glb(reinterpret_cast<uint32_t *>(p)), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(void *p, uint64_t v) {
    __hip_atomic_store(glb(reinterpret_cast<uint64_t *>(p)), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld32(const void *p) {
    return __hip_atomic_load(glb(reinterpret_cast<const uint32_t *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld64(const void *p) {
    return __hip_atomic_load(glb(reinterpret_cast<const uint64_t *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Hand-off words are read with these atomic loads: a plain load can hit a line that the
// reading XCD's L2 still holds from before the write (the L2s of different XCDs are not
// kept coherent). The compiler waits for each atomic load before its first use, so the
// code below issues them in unrolled batches (loads first, uses after): a batch costs
// one memory latency.
__device__ __forceinline__ uint64_t tagged(uint32_t v, uint32_t tag) { return ((uint64_t)tag << 32) | v; }
__device__ __forceinline__ bool current(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

}  // namespace dev
}  // namespace moe
