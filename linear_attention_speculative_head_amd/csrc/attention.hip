// Tree-aware softmax-attention verify on gfx950, the other half of a tree verify pass in a
// Gated DeltaNet hybrid: every draft node's query attends to the committed key/value cache
// plus its own ancestors-or-self among the draft tokens (technical review "TreeWY: Removing
// the Memory Wall in Speculative Decoding for Gated DeltaNet Hybrids", §2.3 "KV cache
// attention", Eq. (2), and §2.2 on tree-structured drafting), with the ancestor sets the GDN
// path uses.  Head dimension 256; query head hq reads key/value head hq / G.
//
// Split over the cache (the HBM stream): one wave per (sequence, key/value head, block of 32
// queries, 512 cache rows).  It keeps the 32 queries in registers as MFMA fragments and walks
// its rows 32 at a time: keys and values HBM -> LDS (global_load_lds_dwordx4), scores
// S = Q K^T on the matrix cores (bf16 inputs, fp32 accumulation), an online softmax in base
// 2, P = exp2(S - m) split into bf16 hi + lo (|P - hi - lo| <= 2^-18 P) and O += P V on the
// matrix cores, rescaled as the running maximum moves.  Its partial (O unnormalised, the row
// maxima m, the row sums l) goes to a workspace.  A second kernel merges the partials of each
// query, adds the draft keys it may see (at most 64, walked from the tree), and normalises.

#include "device_common.h"
#include "launch.h"

namespace treewy {

namespace {

constexpr int DA = 256;                     // head dimension
constexpr int kQB = 32;                     // queries per block (two MFMA row tiles)
constexpr int kTile = 32;                   // cache rows per step
constexpr int kSplit = 512;                 // cache rows per wave
constexpr int kPartFloats = kQB * DA + 2 * kQB;   // O [32][256], m [32], l [32]
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One HBM -> LDS load of 16 bytes per lane (lane l lands at lds + 16 l), from a scalar base and
// a 32-bit lane offset.  M0 holds the LDS destination and is restored; the caller waits on
// vmcnt before reading the rows.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);
    const uint64_t x = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    const void* b = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(b)
        : "memory");
}

__device__ __forceinline__ int clamp_ctx(int c, int T_max) { return c < 0 ? 0 : (c > T_max ? T_max : c); }

// grid (splits, query blocks, B * Hkv), one wave
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1)))
void attn_partial_kernel(const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vc,
                         const int32_t* __restrict__ ctx, int T_max,
                         const uint16_t* __restrict__ Qd, int Hkv, int G, int N,
                         float* __restrict__ work)
{
    __shared__ __align__(16) uint16_t sK[kTile * DA];     // rows 512 B, chunk c at c ^ (r % 16)
    __shared__ __align__(16) uint16_t sV[kTile * DA];     // rows 512 B, plain
    __shared__ __align__(16) uint16_t sP[2][kQB * kTile]; // P hi / lo [32 q][32 rows]

    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int split = blockIdx.x;
    const int qb = blockIdx.y;
    const int bk = blockIdx.z;                  // b * Hkv + kvh
    const int b = bk / Hkv;
    const int kvh = bk - b * Hkv;
    const int Hq = Hkv * G;
    const int Nq = N * G;
    const int c = clamp_ctx(ctx[b], T_max);
    const int k0 = split * kSplit;
    if (k0 >= c) return;                        // nothing of this sequence's cache here
    const int k1 = k0 + kSplit < c ? k0 + kSplit : c;

    // the block's queries as A fragments: lane L holds row L % 16 of tile qt, dims
    // 32 kb + 8 (L / 16) .. +7
    bf16x8_t qf[2][8];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int qi = qb * kQB + 16 * qt + col;
        const bool ok = qi < Nq;
        const int t = ok ? qi / G : 0;
        const int hq = kvh * G + (ok ? qi - t * G : 0);
        const uint16_t* qrow = Qd + (static_cast<size_t>(b * N + t) * Hq + hq) * DA;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            u32x4_t w = {0u, 0u, 0u, 0u};
            if (ok) w = *reinterpret_cast<const u32x4_t*>(qrow + 32 * kb + 8 * grp);
            qf[qt][kb] = __builtin_bit_cast(bf16x8_t, w);
        }
    }

    f32x4_t acc[2][16];                         // O tiles: lane: dim 16 dt + L % 16, rows 4 grp + i
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) acc[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[2][4], l[2][4];                     // per row 4 grp + i of tile qt (base-2 domain)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) { m[qt][i] = -INFINITY; l[qt][i] = 0.f; }

    const uint16_t* Kb = Kc + static_cast<size_t>(bk) * T_max * DA;
    const uint16_t* Vb = Vc + static_cast<size_t>(bk) * T_max * DA;
    const uint32_t ldsK = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sK));
    const uint32_t ldsV = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sV));
    const float sscale = kLog2e / 16.0f;        // 1 / sqrt(256), in base 2
    const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
    const uint32_t ch = static_cast<uint32_t>(lane) & 31u;

    for (int kk = k0; kk < k1; kk += kTile) {
        // rows kk .. kk + 31 (past k1: row kk again, masked below) -> LDS, two rows per load
        __builtin_amdgcn_s_waitcnt(0xC07F);     // every LDS read of the last step is done
#pragma unroll
        for (int i = 0; i < kTile / 2; ++i) {
            const uint32_t r = 2u * i + hl;
            const uint32_t row = kk + r < static_cast<uint32_t>(k1) ? kk + r : kk;
            dma16(Kb, row * (DA * 2u) + 16u * (ch ^ (r & 15u)), ldsK + 1024u * i);
            dma16(Vb, row * (DA * 2u) + 16u * ch, ldsV + 1024u * i);
        }
        __builtin_amdgcn_s_waitcnt(0);

        // scores: lane holds row kk + 16 kt + L % 16 for query rows 4 grp + i of tile qt
        f32x4_t s[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int r = 16 * kt + col;
            bf16x8_t kf[8];
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const int c16 = (4 * kb + grp) ^ (r & 15);
                kf[kb] = __builtin_bit_cast(bf16x8_t,
                                            *reinterpret_cast<const u32x4_t*>(sK + r * DA + 8 * c16));
            }
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[qt][kb], kf[kb], a, 0, 0, 0);
                const bool live = kk + r < k1;
#pragma unroll
                for (int i = 0; i < 4; ++i) s[qt][kt][i] = live ? a[i] * sscale : -INFINITY;
            }
        }

        // online softmax per query row: maxima and sums over the 16 lanes of a group
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float mx = fmaxf(s[qt][0][i], s[qt][1][i]);
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
                const float mn = fmaxf(m[qt][i], mx);          // finite: row kk is live
                const float alpha = __builtin_amdgcn_exp2f(m[qt][i] - mn);
                const float p0 = __builtin_amdgcn_exp2f(s[qt][0][i] - mn);
                const float p1 = __builtin_amdgcn_exp2f(s[qt][1][i] - mn);
                s[qt][0][i] = p0;
                s[qt][1][i] = p1;
                float sum = p0 + p1;
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o);
                l[qt][i] = l[qt][i] * alpha + sum;
                m[qt][i] = mn;
#pragma unroll
                for (int dt = 0; dt < 16; ++dt) acc[qt][dt][i] *= alpha;
            }
        }

        // P -> LDS as bf16 hi and lo [query][row], then back as A fragments (row L % 16,
        // rows of the cache 8 (L / 16) .. +7)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = s[qt][kt][i];
                    const __bf16 ph = static_cast<__bf16>(p);
                    const __bf16 pl = static_cast<__bf16>(p - static_cast<float>(ph));
                    const int q = 16 * qt + 4 * grp + i;
                    const int r = 16 * kt + col;
                    sP[0][q * kTile + r] = __builtin_bit_cast(uint16_t, ph);
                    sP[1][q * kTile + r] = __builtin_bit_cast(uint16_t, pl);
                }
        bf16x8_t pa[2][2];                      // [hi/lo][qt]
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
                pa[h2][qt] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(&sP[h2][(16 * qt + col) * kTile + 8 * grp]));

        // O += P V: B fragments lane L: dim 16 dt + L % 16, cache rows 8 (L / 16) .. +7
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            const int d = 16 * dt + col;
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t e0 = sV[(8 * grp + 2 * j) * DA + d];
                const uint32_t e1 = sV[(8 * grp + 2 * j + 1) * DA + d];
                w[j] = e0 | (e1 << 16);
            }
            const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[0][qt], vf, acc[qt][dt], 0, 0, 0);
                acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[1][qt], vf, acc[qt][dt], 0, 0, 0);
            }
        }
    }

    // the partial: O rows (unnormalised), then m and l
    const int nsplit = (T_max + kSplit - 1) / kSplit;
    const int nqb = (Nq + kQB - 1) / kQB;
    float* part = work + (static_cast<size_t>(bk * nqb + qb) * nsplit + split) * kPartFloats;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int dt = 0; dt < 16; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part[(16 * qt + 4 * grp + i) * DA + 16 * dt + col] = acc[qt][dt][i];
    if (col == 0) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                part[kQB * DA + 16 * qt + 4 * grp + i] = m[qt][i];
                part[kQB * DA + kQB + 16 * qt + 4 * grp + i] = l[qt][i];
            }
    }
}

// grid (query blocks, B * Hkv), 256 lanes: lane = (query row q = tid / 8, dims 32 (tid % 8) ..
// +31).  Merges the cache partials of each query and the draft keys it may see.
__global__ __launch_bounds__(256)
void attn_combine_kernel(const int32_t* __restrict__ ctx, int T_max,
                         const uint16_t* __restrict__ Qd, const uint16_t* __restrict__ Kd,
                         const uint16_t* __restrict__ Vd, const int32_t* __restrict__ parent,
                         int Hkv, int G, int N, const float* __restrict__ work,
                         float* __restrict__ O, int32_t* __restrict__ status)
{
    const int tid = threadIdx.x;
    const int qr = tid >> 3;
    const int dc = (tid & 7) * 32;
    const int qb = blockIdx.x;
    const int bk = blockIdx.y;
    const int b = bk / Hkv;
    const int kvh = bk - b * Hkv;
    const int Hq = Hkv * G;
    const int Nq = N * G;
    const int qi = qb * kQB + qr;
    const bool ok = qi < Nq;                    // every lane takes part in the shuffles
    const int t = ok ? qi / G : 0;
    const int hq = kvh * G + (ok ? qi - t * G : 0);
    const int craw = ctx[b];
    const int c = clamp_ctx(craw, T_max);
    if (tid == 0 && qb == 0 && kvh == 0 && craw != c) report(status, TREEWY_ECTX);
    const int nsplit = (T_max + kSplit - 1) / kSplit;
    const int nqb = (Nq + kQB - 1) / kQB;
    const int used = (c + kSplit - 1) / kSplit;

    // the query's slice and the draft part's scores
    const uint16_t* qrow = Qd + (static_cast<size_t>(b * N + t) * Hq + hq) * DA + dc;
    float q[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) q[e] = bf16_to_f32(qrow[e]);

    float mx = -INFINITY;
    const float* base = work + static_cast<size_t>(bk * nqb + qb) * nsplit * kPartFloats;
    for (int s = 0; s < used; ++s) mx = fmaxf(mx, base[s * kPartFloats + kQB * DA + qr]);

    // ancestors-or-self of t, walked from the tree (a malformed parent ends the walk)
    int node = t;
    float acc[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] = 0.f;
    float lsum = 0.f;
    float dmax = -INFINITY;
    for (int hop = 0; hop < 64 && node >= 0; ++hop) {    // first pass: the draft maximum
        const uint16_t* krow = Kd + (static_cast<size_t>(b * N + node) * Hkv + kvh) * DA + dc;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) part += q[e] * bf16_to_f32(krow[e]);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 4);
        dmax = fmaxf(dmax, part * (kLog2e / 16.0f));
        const int p = parent[b * N + node];
        node = (p >= -1 && p < node) ? p : -1;
    }
    const float mt = fmaxf(mx, dmax);
    for (int s = 0; s < used; ++s) {
        const float* ps = base + s * kPartFloats;
        const float w = __builtin_amdgcn_exp2f(ps[kQB * DA + qr] - mt);
        lsum += w * ps[kQB * DA + kQB + qr];
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] += w * ps[qr * DA + dc + e];
    }
    node = t;
    for (int hop = 0; hop < 64 && node >= 0; ++hop) {    // second pass: the draft terms
        const size_t row = (static_cast<size_t>(b * N + node) * Hkv + kvh) * DA + dc;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) part += q[e] * bf16_to_f32(Kd[row + e]);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 4);
        const float w = __builtin_amdgcn_exp2f(part * (kLog2e / 16.0f) - mt);
        lsum += w;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] += w * bf16_to_f32(Vd[row + e]);
        const int p = parent[b * N + node];
        if (p < -1 || p >= node) {
            if (ok && (tid & 7) == 0) report(status, TREEWY_ETREE);
            node = -1;
        } else {
            node = p;
        }
    }
    if (!ok) return;
    const float inv = 1.0f / lsum;
    float* orow = O + (static_cast<size_t>(b * N + t) * Hq + hq) * DA + dc;
#pragma unroll
    for (int e = 0; e < 32; e += 4)
        *reinterpret_cast<f32x4_t*>(orow + e) = f32x4_t{acc[e] * inv, acc[e + 1] * inv,
                                                         acc[e + 2] * inv, acc[e + 3] * inv};
}

// grid (B * Hkv), 256 lanes: the accepted node's root-to-node path (keys and values of one
// key/value head) appended after the committed prefix; the new length into ctx_out.
__global__ __launch_bounds__(256)
void kv_commit_kernel(uint16_t* __restrict__ Kc, uint16_t* __restrict__ Vc,
                      const int32_t* __restrict__ ctx_in, int32_t* __restrict__ ctx_out,
                      int T_max, const uint16_t* __restrict__ Kd, const uint16_t* __restrict__ Vd,
                      const int32_t* __restrict__ parent, const int32_t* __restrict__ accepted,
                      int Hkv, int N, int32_t* __restrict__ status)
{
    __shared__ int s_path[64];
    __shared__ int s_len;
    const int tid = threadIdx.x;
    const int bk = blockIdx.x;
    const int b = bk / Hkv;
    const int kvh = bk - b * Hkv;
    const int craw = ctx_in[b];
    const int a = accepted[b];
    if (tid == 0) {
        int len = 0;
        bool okp = craw >= 0 && craw <= T_max;
        if (!okp && kvh == 0) report(status, TREEWY_ECTX);
        if (a < -1 || a >= N) {
            if (kvh == 0) report(status, TREEWY_EACCEPT);
            okp = false;
        }
        if (okp && a >= 0) {
            // walk up once for the length (and the tree's validity), then again filling the
            // path root first
            for (int i = a; i >= 0 && len < 64; ++len) {
                const int p = parent[b * N + i];
                if (p < -1 || p >= i) {
                    okp = false;
                    if (kvh == 0) report(status, TREEWY_ETREE);
                    break;
                }
                i = p;
            }
            if (okp && craw + len > T_max) {
                okp = false;
                if (kvh == 0) report(status, TREEWY_ECTX);
            }
            if (okp) {
                int i = a;
                for (int j = len - 1; j >= 0; --j) {
                    s_path[j] = i;
                    i = parent[b * N + i];
                }
            }
        }
        s_len = okp ? len : 0;
        if (kvh == 0) ctx_out[b] = okp ? craw + len : clamp_ctx(craw, T_max);
    }
    __syncthreads();
    const int len = s_len;
    for (int j = 0; j < len; ++j) {
        const size_t src = (static_cast<size_t>(b * N + s_path[j]) * Hkv + kvh) * DA;
        const size_t dst = (static_cast<size_t>(bk) * T_max + craw + j) * DA;
        Kc[dst + tid] = Kd[src + tid];
        Vc[dst + tid] = Vd[src + tid];
    }
}

}  // namespace

size_t attention_workspace_bytes(int B, int Hkv, int G, int N, int T_max) {
    const size_t nsplit = (static_cast<size_t>(T_max) + kSplit - 1) / kSplit;
    const size_t nqb = (static_cast<size_t>(N) * G + kQB - 1) / kQB;
    return static_cast<size_t>(B) * Hkv * nqb * nsplit * kPartFloats * sizeof(float);
}

hipError_t launch_tree_attention(const AttentionArgs& a, hipStream_t stream) {
    const int nsplit = (a.T_max + kSplit - 1) / kSplit;
    const int nqb = (a.N * a.G + kQB - 1) / kQB;
    hipLaunchKernelGGL(attn_partial_kernel, dim3(nsplit, nqb, a.B * a.Hkv), dim3(64), 0, stream,
                       static_cast<const uint16_t*>(a.Kc), static_cast<const uint16_t*>(a.Vc),
                       a.ctx, a.T_max, static_cast<const uint16_t*>(a.Qd), a.Hkv, a.G, a.N,
                       static_cast<float*>(a.work));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(nqb, a.B * a.Hkv), dim3(256), 0, stream, a.ctx,
                       a.T_max, static_cast<const uint16_t*>(a.Qd),
                       static_cast<const uint16_t*>(a.Kd), static_cast<const uint16_t*>(a.Vd),
                       a.parent, a.Hkv, a.G, a.N, static_cast<const float*>(a.work), a.O, a.status);
    return hipGetLastError();
}

hipError_t launch_kv_commit(const KvCommitArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(kv_commit_kernel, dim3(a.B * a.Hkv), dim3(256), 0, stream,
                       static_cast<uint16_t*>(a.Kc), static_cast<uint16_t*>(a.Vc), a.ctx_in,
                       a.ctx_out, a.T_max, static_cast<const uint16_t*>(a.Kd),
                       static_cast<const uint16_t*>(a.Vd), a.parent, a.accepted, a.Hkv, a.N,
                       a.status);
    return hipGetLastError();
}

}  // namespace treewy
