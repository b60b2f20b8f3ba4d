// Device helpers shared by the TreeWY kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treewy.h"

namespace treewy {

constexpr int D = 128;       // dk = dv
constexpr int MAXN = 64;     // one uint64 ancestor mask per node

// bfloat16 is carried as its 16-bit pattern; widening to float is exact.
__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    // 4 consecutive elements starting at p (p 16-byte aligned)
    static __device__ __forceinline__ float4 load4(const float* p) {
        return *reinterpret_cast<const float4*>(p);
    }
    static __device__ __forceinline__ float load1(const float* p) { return *p; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float4 load4(const uint16_t* p) {
        uint2 w = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    }
    static __device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }
};

__device__ __forceinline__ float dot4(float4 a, float4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
    uint32_t lo = __shfl(static_cast<uint32_t>(x), src);
    uint32_t hi = __shfl(static_cast<uint32_t>(x >> 32), src);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Workgroup barrier that orders LDS only: every wave's LDS writes before it are visible to
// every wave after it, while global loads and stores stay in flight (a plain __syncthreads
// also waits for all outstanding global memory operations).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void report(int32_t* status, int code) {
    if (status) atomicCAS(reinterpret_cast<int*>(status), 0, code);
}

// Tree bookkeeping for one draft tree, run by all 64 lanes of one wave (lane t = node t).
// Pointer jumping: after round r every lane holds the set of its ancestors at distance
// < 2^r (itself included) and the product of their gates, plus a pointer to the ancestor
// at distance 2^r.  Parents precede their children, so a node's depth is at most N and
// ceil(log2 N) rounds cover every ancestor (six for 64 nodes).  A parent outside
// [-1, t-1] is reported and treated as -1 so that every later index stays in range.
struct NodeInfo {
    uint64_t anc;   // inclusive ancestor mask
    float g;        // product of the gates on the path (1 for lanes >= N)
    int depth;
    bool bad;
};

__device__ __forceinline__ NodeInfo tree_walk(const int32_t* parent_b, int N, float alpha_t) {
    const int lane = threadIdx.x & 63;
    int p = -1;
    bool bad = false;
    if (lane < N) {
        p = parent_b[lane];
        if (p < -1 || p >= lane) { bad = true; p = -1; }
    }
    uint64_t a = lane < N ? (1ull << lane) : 0ull;
    float g = lane < N ? alpha_t : 1.0f;
    int j = p;
    for (int r = 0; (1 << r) < N; ++r) {
        const int src = j < 0 ? lane : j;
        const uint64_t aj = shfl_u64(a, src);
        const float gj = __shfl(g, src);
        const int jj = __shfl(j, src);
        if (j >= 0) { a |= aj; g *= gj; j = jj; }
    }
    NodeInfo n;
    n.anc = a;
    n.g = g;
    n.depth = __popcll(a);
    n.bad = bad;
    return n;
}

}  // namespace treewy
