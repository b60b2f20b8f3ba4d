// Full-state snapshotting ("store-all"), the comparison scheme of the TreeWY paper
// (arXiv 2608.20961, §2 "The memory problem", approach (i)): every draft node's state is
// materialised, and rollback copies the accepted node's snapshot.
//
// Verify: one workgroup per (sequence, head).  Each wave owns 32 rows of the state, each
// half-wave one row at a time with a float4 of columns per lane, so every snapshot row is
// written with full 512-byte coalesced stores.  Nodes run in index order (parents first);
// node t applies Eq. (1) row by row to its parent's state:
//     S_t[r,:] = a_t S_p[r,:] + (b_t v_t[r] - a_t b_t (S_p[r,:] . k_t)) k_t^T,
//     o_t[r]   = S_t[r,:] . q_t.
// The parent's state is the one just computed when parent(t) = t-1 (kept in registers);
// otherwise each lane re-reads exactly the elements it wrote itself into Snap[parent], or
// S0 for a child of the committed state.

#include "device_common.h"
#include "launch.h"

namespace treewy {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;   // rows per lane: wave w covers rows 32w .. 32w+31, two per step

__device__ __forceinline__ float half_wave_sum(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 8);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 1);
    return x;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void snapshot_verify_kernel(
    const float* __restrict__ S0, const T* __restrict__ Q, const T* __restrict__ K,
    const T* __restrict__ V, const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ parent, int H, int N, float* __restrict__ O,
    float* __restrict__ Snap, int32_t* __restrict__ status)
{
    __shared__ int s_par[MAXN];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c4 = lane & 31;
    const int row0 = wave * 32 + (lane >> 5);     // rows row0 + 2m, m = 0..15

    if (tid < N) {
        int p = parent[node0 + tid];
        if (p < -1 || p >= tid) { report(status, TREEWY_ETREE); p = -1; }
        s_par[tid] = p;
    }
    __syncthreads();

    const size_t DD = static_cast<size_t>(D) * D;
    const float* s0 = S0 + bh * DD;
    float* snap_h = Snap + static_cast<size_t>(bh) * N * DD;
    float4 cur[kRows];

    for (int t = 0; t < N; ++t) {
        const int p = s_par[t];
        if (t == 0 || p != t - 1) {
            const float* src = p < 0 ? s0 : snap_h + p * DD;
#pragma unroll
            for (int m = 0; m < kRows; ++m)
                cur[m] = *reinterpret_cast<const float4*>(src + (row0 + 2 * m) * D + 4 * c4);
        }
        const size_t row = (node0 + t) * H + h;
        const float4 k4 = Elem<T>::load4(K + row * D + 4 * c4);
        const float4 q4 = Elem<T>::load4(Q + row * D + 4 * c4);
        const float a_t = alpha[row];
        const float b_t = beta[row];
        float* dst = snap_h + t * DD;
#pragma unroll
        for (int m = 0; m < kRows; ++m) {
            const int r = row0 + 2 * m;
            const float u = half_wave_sum(dot4(cur[m], k4));
            const float vr = Elem<T>::load1(V + row * D + r);
            const float coef = b_t * vr - a_t * b_t * u;
            float4 s = cur[m];
            s.x = a_t * s.x + coef * k4.x;
            s.y = a_t * s.y + coef * k4.y;
            s.z = a_t * s.z + coef * k4.z;
            s.w = a_t * s.w + coef * k4.w;
            cur[m] = s;
            const float o = half_wave_sum(dot4(s, q4));
            *reinterpret_cast<float4*>(dst + r * D + 4 * c4) = s;
            if (c4 == 0) O[row * D + r] = o;
        }
    }
}

__global__ __launch_bounds__(kThreads) void snapshot_commit_kernel(
    float* __restrict__ S, const float* __restrict__ Snap, const int32_t* __restrict__ accepted,
    int H, int N, int32_t* __restrict__ status)
{
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int h = bh - b * H;
    const int a = accepted[b];
    if (a < -1 || a >= N) {
        if (threadIdx.x == 0 && h == 0) report(status, TREEWY_EACCEPT);
        return;
    }
    if (a < 0) return;
    const size_t DD = static_cast<size_t>(D) * D;
    const float4* src = reinterpret_cast<const float4*>(Snap + (static_cast<size_t>(bh) * N + a) * DD);
    float4* dst = reinterpret_cast<float4*>(S + static_cast<size_t>(bh) * DD);
    float4 x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = src[j * kThreads + threadIdx.x];
#pragma unroll
    for (int j = 0; j < 16; ++j) dst[j * kThreads + threadIdx.x] = x[j];
}

}  // namespace

template <typename T>
static hipError_t launch_snapshot_verify_t(const SnapshotVerifyArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(snapshot_verify_kernel<T>, dim3(a.B * a.H), dim3(kThreads), 0, stream,
                       a.S0, static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                       static_cast<const T*>(a.V), a.alpha, a.beta, a.parent, a.H, a.N, a.O,
                       a.Snap, a.status);
    return hipGetLastError();
}

hipError_t launch_verify_snapshot(const SnapshotVerifyArgs& a, hipStream_t stream) {
    return a.in_dtype == TREEWY_BF16 ? launch_snapshot_verify_t<uint16_t>(a, stream)
                                     : launch_snapshot_verify_t<float>(a, stream);
}

hipError_t launch_commit_snapshot(const SnapshotCommitArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(snapshot_commit_kernel, dim3(a.B * a.H), dim3(kThreads), 0, stream, a.S,
                       a.Snap, a.accepted, a.H, a.N, a.status);
    return hipGetLastError();
}

}  // namespace treewy
