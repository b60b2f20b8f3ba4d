// TreeWY commit on gfx950: rebuild the accepted node's state in place.
//
// Paper: "TreeWY: Speculative Verification for Gated DeltaNet Hybrids" (arXiv 2608.20961),
// §3 "Reconstruct on commit", Eq. (3):  S_a = g_a S0 + sum over i ancestor-or-self of a
// of (g_a/g_i) vt~_i k_i^T.  Only the pseudo-values U (one 128-row per node), the keys and
// the cumulative gates of a's path are needed; no per-node state exists.
//
// One workgroup of 256 lanes per (sequence, head, half of the rows).  The state is a pure
// HBM stream: every lane issues its 8 float4 loads of S at once, the path (at most 64
// nodes) is walked in LDS while they are in flight, the rank-depth(a) update is applied in
// registers and S is written back.  a = -1 exits before touching S.

#include "device_common.h"
#include "launch.h"

namespace treewy {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;                        // path rows staged per pass
constexpr int kParts = 2;                         // row slices per head
constexpr int kVec = D * D / 4 / kThreads / kParts;  // float4 of S per lane (8)

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// State rows with the non-temporal (streaming) hint: the commit reads each row once and
// overwrites it, so neither the read nor the written lines are worth keeping in the caches.
__device__ __forceinline__ float4 load_stream(const float4* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(float4* p, float4 x) {
    __builtin_nontemporal_store(f32x4_t{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4_t*>(p));
}

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5)))
void commit_kernel(
    float* __restrict__ S, const float* __restrict__ U, const T* __restrict__ K,
    const float* __restrict__ gamma, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ accepted, int H, int N, int32_t* __restrict__ status)
{
    __shared__ int s_par[MAXN];
    __shared__ int s_path[MAXN];
    __shared__ int s_len;
    __shared__ float s_cu[kChunk][D];   // (g_a/g_i) U[i]
    __shared__ float s_k[kChunk][D];    // k_i

    const int tid = threadIdx.x;
    const int bh = blockIdx.x / kParts;
    const int part = blockIdx.x - bh * kParts;
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;

    const int a = accepted[b];
    if (a < -1 || a >= N) {
        if (tid == 0 && h == 0 && part == 0) report(status, TREEWY_EACCEPT);
        return;
    }
    if (a < 0) return;

    // issue the state loads first; they do not depend on the path
    constexpr int kRowsPart = D / kParts;
    float4* Sh = reinterpret_cast<float4*>(S + (static_cast<size_t>(bh) * D + part * kRowsPart) * D);
    float4 s[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) s[j] = load_stream(&Sh[j * kThreads + tid]);

    if (tid < N) s_par[tid] = parent[node0 + tid];
    __syncthreads();
    if (tid == 0) {
        int len = 0;
        int i = a;
        bool ok = true;
        while (i >= 0) {
            s_path[len++] = i;
            const int p = s_par[i];
            if (p < -1 || p >= i) { ok = false; break; }
            i = p;
        }
        s_len = ok ? len : -1;
        if (!ok && h == 0 && part == 0) report(status, TREEWY_ETREE);
    }
    __syncthreads();
    const int len = s_len;
    if (len < 0) return;                      // malformed tree: leave S untouched

    const float ga = gamma[(node0 + a) * H + h];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        s[j].x *= ga; s[j].y *= ga; s[j].z *= ga; s[j].w *= ga;
    }

    const int c4 = tid & 31;                  // this lane's 4 columns: 4*c4 .. 4*c4+3
    for (int c0 = 0; c0 < len; c0 += kChunk) {
        const int nj = min(kChunk, len - c0);
        __syncthreads();
        for (int p = tid; p < nj * D; p += kThreads) {
            const int jj = p >> 7;
            const int x = p & (D - 1);
            const int i = s_path[c0 + jj];
            const size_t row = ((node0 + i) * H + h) * D;
            const float coef = ga / gamma[(node0 + i) * H + h];
            s_cu[jj][x] = coef * U[row + x];   // only this part's rows are used
            s_k[jj][x] = Elem<T>::load1(K + row + x);
        }
        __syncthreads();
#pragma unroll 1
        for (int jj = 0; jj < nj; ++jj) {
            const float4 kv = *reinterpret_cast<const float4*>(&s_k[jj][4 * c4]);
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const int r = part * kRowsPart + ((j * kThreads + tid) >> 5);
                const float cu = s_cu[jj][r];
                s[j].x += cu * kv.x; s[j].y += cu * kv.y; s[j].z += cu * kv.z; s[j].w += cu * kv.w;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kVec; ++j) store_stream(&Sh[j * kThreads + tid], s[j]);
}

// The state a deferred-commit log stands for, written back: S <- scale (S + sum_j u~_j k_j^T)
// for the first len[b] terms, and the log emptied (scale 1, length 0 into the output
// header).  Same work split as commit_kernel; an empty log leaves S untouched.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5)))
void flush_kernel(
    float* __restrict__ S, const float* __restrict__ logU, const uint16_t* __restrict__ logK,
    const float* __restrict__ scale_in, float* __restrict__ scale_out,
    const int32_t* __restrict__ len_in, int32_t* __restrict__ len_out, int H, int Lmax,
    int32_t* __restrict__ status)
{
    __shared__ float s_u[kChunk][D / kParts];   // this half's rows of u~
    __shared__ float s_k[kChunk][D];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x / kParts;
    const int part = blockIdx.x - bh * kParts;
    const int b = bh / H;
    const int h = bh - b * H;

    const int raw = len_in[b];
    const int len = raw < 0 ? 0 : (raw > Lmax ? Lmax : raw);
    if (tid == 0 && part == 0) {
        if (raw != len && h == 0) report(status, TREEWY_ELOG);
        scale_out[bh] = 1.0f;
        if (h == 0) len_out[b] = 0;
    }
    if (len == 0) return;                     // an empty log: S is the state already
    const float sc = scale_in[bh];

    constexpr int kRowsPart = D / kParts;
    float4* Sh = reinterpret_cast<float4*>(S + (static_cast<size_t>(bh) * D + part * kRowsPart) * D);
    float4 s[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) s[j] = Sh[j * kThreads + tid];

    const size_t row0 = static_cast<size_t>(bh) * Lmax;
    const int c4 = tid & 31;
    for (int c0 = 0; c0 < len; c0 += kChunk) {
        const int nj = min(kChunk, len - c0);
        __syncthreads();
        for (int p = tid; p < nj * D; p += kThreads) {
            const int jj = p >> 7;
            const int x = p & (D - 1);
            if (x < kRowsPart) s_u[jj][x] = logU[(row0 + c0 + jj) * D + part * kRowsPart + x];
            s_k[jj][x] = Elem<uint16_t>::load1(logK + (row0 + c0 + jj) * D + x);
        }
        __syncthreads();
#pragma unroll 1
        for (int jj = 0; jj < nj; ++jj) {
            const float4 kv = *reinterpret_cast<const float4*>(&s_k[jj][4 * c4]);
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const int r = (j * kThreads + tid) >> 5;
                const float cu = s_u[jj][r];
                s[j].x += cu * kv.x; s[j].y += cu * kv.y; s[j].z += cu * kv.z; s[j].w += cu * kv.w;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        s[j].x *= sc; s[j].y *= sc; s[j].z *= sc; s[j].w *= sc;
        Sh[j * kThreads + tid] = s[j];
    }
}

}  // namespace

hipError_t launch_deferred_flush(float* S, const DeferArgs& d, int B, int H, int in_dtype,
                                 int32_t* status, hipStream_t stream) {
    (void)in_dtype;                           // the log's keys are bf16
    hipLaunchKernelGGL(flush_kernel, dim3(B * H * kParts), dim3(kThreads), 0, stream, S, d.logU,
                       static_cast<const uint16_t*>(d.logK), d.scale_in, d.scale_out, d.len_in,
                       d.len_out, H, d.Lmax, status);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_commit_t(const CommitArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(commit_kernel<T>, dim3(a.B * a.H * kParts), dim3(kThreads), 0, stream, a.S, a.U,
                       static_cast<const T*>(a.K), a.gamma, a.parent, a.accepted, a.H, a.N,
                       a.status);
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t stream) {
    return a.in_dtype == TREEWY_BF16 ? launch_commit_t<uint16_t>(a, stream)
                                     : launch_commit_t<float>(a, stream);
}

}  // namespace treewy
