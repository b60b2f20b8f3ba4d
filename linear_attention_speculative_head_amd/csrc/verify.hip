// TreeWY tree verification on gfx950.
//
// Paper: "TreeWY: Speculative Verification for Gated DeltaNet Hybrids" (arXiv 2608.20961),
// §3 "Verifying a draft", Eq. (2), and the per-node readout o_t = S_t q_t with S_t written
// through the unrolled form of §3 "Reconstruct on commit" (Eq. 3 evaluated at a = t).
//
// One workgroup of 256 lanes per (sequence, head):
//   1. tree walk (one wave, pointer jumping): ancestor masks, depths, cumulative gates g_t;
//      the ancestor pairs (t, i), i ancestor-or-self of t, are listed root first;
//   2. the S0 stream: P[t] = S0 k_t and Y[t] = S0 q_t, S0 read once from HBM (lane = row v);
//   3. R[t] = b_t (v_t - g_t P[t]);  coefficients on ancestor pairs only:
//      C = b_t (g_t/g_i)(k_t . k_i) for strict ancestors, W = (g_t/g_i)(k_i . q_t);
//   4. forward substitution U[t] = R[t] - sum_i C[t,i] U[i] in node order (parents first),
//      one lane per value column v (columns are independent);
//   5. readout O[t] = g_t Y[t] + sum_{i anc-or-self} W[t,i] U[i]; O, U, gamma written once.

#include "device_common.h"
#include "launch.h"

namespace treewy {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxPairs = MAXN * (MAXN + 1) / 2;  // a chain of 64 nodes

struct VerifyShared {
    uint64_t anc[MAXN];
    float g[MAXN];
    float beta[MAXN];
    int depth[MAXN];
    int base[MAXN + 1];          // first pair of node t; base[N] = number of pairs
    uint8_t pair_t[kMaxPairs];
    uint8_t pair_i[kMaxPairs];
    float pair_c[kMaxPairs];     // b_t (g_t/g_i)(k_t . k_i); 0 on the diagonal pair
    float pair_w[kMaxPairs];     // (g_t/g_i)(k_i . q_t)
};

template <typename T>
__global__ __launch_bounds__(kThreads) void verify_kernel(
    const float* __restrict__ S0, const T* __restrict__ Q, const T* __restrict__ K,
    const T* __restrict__ V, const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ parent, int H, int N, float* __restrict__ O,
    float* __restrict__ U, float* __restrict__ gamma, uint64_t* __restrict__ anc_out,
    int32_t* __restrict__ depth_out, int32_t* __restrict__ status)
{
    __shared__ VerifyShared sh;
    extern __shared__ float dyn[];
    float* P = dyn;                 // [N][128]: S0 k_t, then R, then U
    float* Y = dyn + N * D;         // [N][128]: S0 q_t

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;   // row (b, t=0) of [B, N, ...]

    // ---- 1. tree walk (wave 0)
    if (tid < 64) {
        const int t = tid;
        const size_t nh = (node0 + t) * H + h;
        const float a_t = t < N ? alpha[nh] : 1.0f;
        NodeInfo ni = tree_walk(parent + node0, N, a_t);
        if (ni.bad) report(status, TREEWY_ETREE);
        // exclusive prefix sum of depths -> first pair index of each node
        int incl = t < N ? ni.depth : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (t >= off) incl += y;
        }
        if (t < N) {
            const int start = incl - ni.depth;
            sh.anc[t] = ni.anc;
            sh.g[t] = ni.g;
            sh.beta[t] = beta[nh];
            sh.depth[t] = ni.depth;
            sh.base[t] = start;
            uint64_t m = ni.anc;
            int idx = start;
            while (m) {                       // ancestors in increasing index = root first
                const int i = __ffsll(static_cast<unsigned long long>(m)) - 1;
                m &= m - 1;
                sh.pair_t[idx] = static_cast<uint8_t>(t);
                sh.pair_i[idx] = static_cast<uint8_t>(i);
                ++idx;
            }
            gamma[nh] = ni.g;
            if (h == 0) {
                if (anc_out) anc_out[node0 + t] = ni.anc;
                if (depth_out) depth_out[node0 + t] = ni.depth;
            }
        }
        if (t == N - 1) sh.base[N] = incl;
    }

    // ---- 2. S0 stream: lane v owns row v; the two lane halves take alternate node groups
    {
        const int v = tid & (D - 1);
        const int half = tid >> 7;
        const float* srow = S0 + (static_cast<size_t>(bh) * D + v) * D;
        for (int t0 = half * 4; t0 < N; t0 += 8) {
            float pk[4] = {0.f, 0.f, 0.f, 0.f};
            float pq[4] = {0.f, 0.f, 0.f, 0.f};
            const int nt = min(4, N - t0);
            for (int c = 0; c < D; c += 4) {
                const float4 s = *reinterpret_cast<const float4*>(srow + c);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (j < nt) {
                        const size_t row = ((node0 + t0 + j) * H + h) * D + c;
                        pk[j] += dot4(s, Elem<T>::load4(K + row));
                        pq[j] += dot4(s, Elem<T>::load4(Q + row));
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < nt) {
                    P[(t0 + j) * D + v] = pk[j];
                    Y[(t0 + j) * D + v] = pq[j];
                }
            }
        }
    }
    __syncthreads();

    // ---- 3a. right-hand side R[t] = b_t (v_t - g_t P[t]), in place
    for (int p = tid; p < N * D; p += kThreads) {
        const int t = p >> 7;
        const int v = p & (D - 1);
        const float vt = Elem<T>::load1(V + ((node0 + t) * H + h) * D + v);
        P[p] = sh.beta[t] * (vt - sh.g[t] * P[p]);
    }
    // ---- 3b. coefficients on ancestor pairs
    const int npairs = sh.base[N];
    for (int p = tid; p < npairs; p += kThreads) {
        const int t = sh.pair_t[p];
        const int i = sh.pair_i[p];
        const T* kt = K + ((node0 + t) * H + h) * D;
        const T* ki = K + ((node0 + i) * H + h) * D;
        const T* qt = Q + ((node0 + t) * H + h) * D;
        float kk = 0.f, kq = 0.f;
        for (int c = 0; c < D; c += 4) {
            const float4 a = Elem<T>::load4(ki + c);
            kk += dot4(a, Elem<T>::load4(kt + c));
            kq += dot4(a, Elem<T>::load4(qt + c));
        }
        const float ratio = sh.g[t] / sh.g[i];
        sh.pair_c[p] = (i == t) ? 0.f : sh.beta[t] * ratio * kk;
        sh.pair_w[p] = ratio * kq;
    }
    __syncthreads();

    // ---- 4. forward substitution, parents before children; lane = value column
    if (tid < D) {
        const int v = tid;
        for (int t = 0; t < N; ++t) {
            float r = P[t * D + v];
            const int p0 = sh.base[t];
            const int p1 = p0 + sh.depth[t] - 1;     // last pair is (t, t)
            for (int p = p0; p < p1; ++p) r -= sh.pair_c[p] * P[sh.pair_i[p] * D + v];
            P[t * D + v] = r;
        }
    }
    __syncthreads();

    // ---- 5. readout and write-out
    for (int p = tid; p < N * D; p += kThreads) {
        const int t = p >> 7;
        const int v = p & (D - 1);
        float o = sh.g[t] * Y[p];
        const int p0 = sh.base[t];
        const int p1 = p0 + sh.depth[t];
        for (int q = p0; q < p1; ++q) o += sh.pair_w[q] * P[sh.pair_i[q] * D + v];
        const size_t out = ((node0 + t) * H + h) * D + v;
        O[out] = o;
        U[out] = P[p];
    }
}

}  // namespace

template <typename T>
static hipError_t launch_verify_t(const VerifyArgs& a, hipStream_t stream) {
    const size_t dyn = static_cast<size_t>(2) * a.N * D * sizeof(float);
    auto kern = verify_kernel<T>;
    if (dyn + sizeof(VerifyShared) > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(dyn));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(kThreads), dyn, stream, a.S0,
                       static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                       static_cast<const T*>(a.V), a.alpha, a.beta, a.parent, a.H, a.N, a.O,
                       a.U, a.gamma, a.anc_out, a.depth_out, a.status);
    return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    return a.in_dtype == TREEWY_BF16 ? launch_verify_t<uint16_t>(a, stream)
                                     : launch_verify_t<float>(a, stream);
}

}  // namespace treewy
