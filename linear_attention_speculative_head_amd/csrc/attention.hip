// Tree-aware softmax-attention verify on gfx950, the other half of a tree verify pass in a
// Gated DeltaNet hybrid: every draft node's query attends to the committed key/value cache
// plus its own ancestors-or-self among the draft tokens (technical review "TreeWY: Removing
// the Memory Wall in Speculative Decoding for Gated DeltaNet Hybrids", §2.3 "KV cache
// attention", Eq. (2), and §2.2 on tree-structured drafting), with the ancestor sets the GDN
// path uses.  Head dimension 256; query head hq reads key/value head hq / G.
//
// Split over the cache (the HBM stream): one workgroup of two waves per (sequence, key/value
// head, block of 32 queries, range of cache rows), the ranges sized at launch so that about
// four workgroups per compute unit cover the batch (few ranges keep the partials' traffic
// small).  Each wave keeps its 16 queries in registers as MFMA fragments; the two walk the
// range's rows 32 at a time, keys and values HBM -> LDS (global_load_lds_dwordx4) in two
// stages so that the next tile's keys stream in while this tile's values are used and the
// next tile's values while the next scores are formed.  Scores are formed transposed, S^T = K Q^T (bf16
// inputs, fp32 accumulation on the matrix cores), so that each lane holds one query's scores
// for 8 cache rows: exactly the B operand the product O^T += V^T P^T needs, so P never leaves
// the registers; it is split into bf16 hi + lo (|P - hi - lo| <= 2^-16 P).  V^T comes from LDS
// with the transposing read of gfx950 (ds_read_b64_tr_b16).  The online softmax (base 2)
// rescales lazily: the running maximum moves only when a score exceeds it by more than 8, so
// P stays below 2^8 and the accumulators are touched only when the maximum really moves; the
// scale cancels in the final normalisation.  The partial (O unnormalised, the row maxima m,
// the row sums l) goes to a workspace.  A second kernel merges the partials of each query,
// adds the draft keys it may see (its ancestors-or-self, at most 64, from the whole tree by
// pointer jumping), and normalises.

#include "device_common.h"
#include "launch.h"

#include <atomic>
#include <mutex>

namespace treewy {

namespace {

constexpr int DA = 256;                     // head dimension
constexpr int kQB = 32;                     // queries per block (two MFMA column tiles)
constexpr int kTile = 32;                   // cache rows per step
constexpr int kTargetBlocks = 640;          // split the cache until about this many workgroups
constexpr int kMinSplit = 256;              // but keep at least this many rows per split
constexpr int kPartFloats = kQB * DA + 2 * kQB;   // O [32][256], m [32], l [32]
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;               // rescale when a score passes the maximum by this

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// s_waitcnt immediates: vector-memory count at most 8 (one stage of a tile still in flight)
// or 0; LDS/scalar and export counts left free.
constexpr int kWaitVm8 = 8 | (7 << 4) | (15 << 8);
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);
constexpr int kWaitLgkm0 = 0xC07F;

// One HBM -> LDS load of 16 bytes per lane (lane l lands at lds + 16 l), from a scalar base and
// a 32-bit lane offset.  M0 holds the LDS destination and is restored; the caller waits on
// vmcnt before reading the rows.  With NT the load carries the non-temporal (streaming) hint:
// for cache rows that only one workgroup of the call reads, so they do not displace other
// data in the caches.
template <bool NT>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);
    const uint64_t x = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    const void* b = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
    uint32_t save;
    if constexpr (NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, %3 nt\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(save)
            : "s"(lds), "v"(voff), "s"(b)
            : "memory");
    else
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

// This wave's half of 32 rows kk .. kk + 31 of one cache (wave w: rows 16 w .. 16 w + 15;
// rows at or past k1 fetch row kk again, their scores are masked) into LDS: row r is 512
// bytes, its 16-byte chunk c stored at position c ^ (r % 16).  Two rows per load, eight loads.
// `stream`: no other query block reads these rows (one block per sequence and head).
__device__ __forceinline__ void load_half(const uint16_t* base, int kk, int k1, uint32_t lds,
                                          int lane, int w, bool stream) {
    const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
    const uint32_t ch = static_cast<uint32_t>(lane) & 31u;
#pragma unroll
    for (int i = 0; i < kTile / 4; ++i) {
        const uint32_t r = 16u * w + 2u * i + hl;
        const uint32_t row = kk + r < static_cast<uint32_t>(k1) ? kk + r : kk;
        const uint32_t off = row * (DA * 2u) + 16u * (ch ^ (r & 15u));
        if (stream)
            dma16<true>(base, off, lds + 8192u * w + 1024u * i);
        else
            dma16<false>(base, off, lds + 8192u * w + 1024u * i);
    }
}

__device__ __forceinline__ int clamp_ctx(int c, int T_max) { return c < 0 ? 0 : (c > T_max ? T_max : c); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(a))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(b))) << 16);
}

// grid (splits, query blocks, B * Hkv), two waves sharing each tile of keys and values: wave w
// owns queries 16 w .. 16 w + 15 of the block and loads rows 16 w .. 16 w + 15 of every tile.
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2)))
void attn_partial_kernel(const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vc,
                         const int32_t* __restrict__ ctx, int T_max,
                         const uint16_t* __restrict__ Qd, int Hkv, int G, int N, int rows,
                         float* __restrict__ work)
{
    __shared__ __align__(16) uint16_t sK[kTile * DA];
    __shared__ __align__(16) uint16_t sV[kTile * DA];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int k0 = split * rows;
    if (k0 >= c) return;                        // nothing of this sequence's cache here (both waves)
    const int k1 = c - k0 > rows ? k0 + rows : c;
    const bool active = qb * kQB + 16 * w < Nq; // wave-uniform: has at least one query

    const uint16_t* Kb = Kc + static_cast<size_t>(bk) * T_max * DA;
    const uint16_t* Vb = Vc + static_cast<size_t>(bk) * T_max * DA;
    const uint32_t ldsK = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sK));
    const uint32_t ldsV = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sV));
    const bool stream = gridDim.y == 1;         // one query block: each row is read once
    load_half(Kb, k0, k1, ldsK, lane, w, stream);
    load_half(Vb, k0, k1, ldsV, lane, w, stream);

    // this wave's queries as B fragments: lane L holds query 16 w + L % 16 of the block, dims
    // 32 kb + 8 (L / 16) .. +7
    bf16x8_t qf[8];
    {
        const int qi = qb * kQB + 16 * w + col;
        const bool ok = qi < Nq;
        const int t = ok ? qi / G : 0;
        const int hq = kvh * G + (ok ? qi - t * G : 0);
        const uint16_t* qrow = Qd + (static_cast<size_t>(b * N + t) * Hq + hq) * DA;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (ok) v = *reinterpret_cast<const u32x4_t*>(qrow + 32 * kb + 8 * grp);
            qf[kb] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    f32x4_t acc[16];                            // O^T tiles: lane: query 16 w + L % 16,
                                                // dims 16 dt + 4 (L / 16) + i
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;                        // running maximum of this lane's query
    float l = 0.f;                              // this lane's share of its row sum
    const float sscale = kLog2e / 16.0f;        // 1 / sqrt(256), in base 2

    // transposing V read: lane (g, i) supplies row 4 g + i / 4 (+16), dims 4 (i % 4) .. +3 of
    // the dim tile; it receives dim i of rows 4 g + j (+16), j = 0..3
    const int vrow = 4 * grp + (col >> 2);
    const uint32_t vsub = 8u * (col & 1);
    const uint32_t vhalf = (col & 3) >> 1;

    for (int kk = k0; kk < k1; kk += kTile) {
        const bool more = kk + kTile < k1;
        // this tile's keys: this wave's loads landed (its value loads may remain), then the
        // other wave's
        __builtin_amdgcn_s_waitcnt(kWaitVm8);
        __syncthreads();

        f32x4_t st[2];                          // S^T: query 16 w + L % 16, rows kk + 16 kt + 4 (L / 16) + i
        if (active) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int r = 16 * kt + col;
                bf16x8_t kf[8];
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    const int c16 = (4 * kb + grp) ^ col;
                    kf[kb] = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const u32x4_t*>(sK + r * DA + 8 * c16));
                }
                f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb], qf[kb], a, 0, 0, 0);
                st[kt] = a;
            }
        }
        // both waves are done with the keys: the next ones stream in during this tile
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __syncthreads();
        if (more) load_half(Kb, kk + kTile, k1, ldsK, lane, w, stream);

        bf16x8_t ph, pl;
        if (active) {
            // scores, masks and the tile maximum of each query
            float v = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool live = kk + 16 * kt + 4 * grp + i < k1;
                    const float sc = live ? st[kt][i] * sscale : -INFINITY;
                    st[kt][i] = sc;
                    v = fmaxf(v, sc);
                }
            v = fmaxf(v, __shfl_xor(v, 16));
            v = fmaxf(v, __shfl_xor(v, 32));    // finite: row kk is live
            if (__any(v > m + kLazy)) {
                const float mn = v > m + kLazy ? v : m;
                const float alpha = __builtin_amdgcn_exp2f(m - mn);     // 0 on the first tile
                m = mn;
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < 16; ++dt) acc[dt] *= alpha;
            }
            // P^T as B fragments: k slots 0..3 = rows 4 g + 0..3, 4..7 = rows 16 + 4 g + 0..3
            float p[8];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[4 * kt + i] = __builtin_amdgcn_exp2f(st[kt][i] - m);
            u32x4_t hw, lw;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hw[j] = pack_bf16(p[2 * j], p[2 * j + 1]);
                const float h0 = __builtin_bit_cast(float, hw[j] << 16);
                const float h1 = __builtin_bit_cast(float, hw[j] & 0xffff0000u);
                lw[j] = pack_bf16(p[2 * j] - h0, p[2 * j + 1] - h1);
            }
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += p[j];
            l += sum;
            ph = __builtin_bit_cast(bf16x8_t, hw);
            pl = __builtin_bit_cast(bf16x8_t, lw);
        }

        // this tile's values: this wave's loads landed (the next keys may remain), then the
        // other wave's
        if (more) __builtin_amdgcn_s_waitcnt(kWaitVm8);
        else __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();

        if (active) {
            // O^T += V^T P^T: A fragments lane (g, i): dim 16 dt + i, cache rows as the k slots
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) {
                const uint32_t chunk = 2u * dt + vhalf;
                const uint32_t a0 = ldsV + vrow * 512u + 16u * (chunk ^ static_cast<uint32_t>(vrow & 15)) + vsub;
                const uint32_t a1 = a0 + 16u * 512u;    // rows + 16: same position (row % 16)
                const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    reinterpret_cast<lds_i16x4_t*>(static_cast<uintptr_t>(a0)));
                const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    reinterpret_cast<lds_i16x4_t*>(static_cast<uintptr_t>(a1)));
                const u32x2_t w0 = __builtin_bit_cast(u32x2_t, t0);
                const u32x2_t w1 = __builtin_bit_cast(u32x2_t, t1);
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, acc[dt], 0, 0, 0);
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, acc[dt], 0, 0, 0);
            }
        }
        // both waves are done with the values: the next ones stream in during the next scores
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __syncthreads();
        if (more) load_half(Vb, kk + kTile, k1, ldsV, lane, w, stream);
    }
    if (!active) return;

    // the partial: O rows (unnormalised), then m and l (l summed over the four lanes that share
    // a query)
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int nsplit = gridDim.x;
    const int nqb = (Nq + kQB - 1) / kQB;
    float* part = work + (static_cast<size_t>(bk * nqb + qb) * nsplit + split) * kPartFloats;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
        *reinterpret_cast<f32x4_t*>(part + (16 * w + col) * DA + 16 * dt + 4 * grp) = acc[dt];
    if (grp == 0) {
        part[kQB * DA + 16 * w + col] = m;
        part[kQB * DA + kQB + 16 * w + col] = l;
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// grid (query groups of 4, B * Hkv), 256 lanes: one wave per query, lane l holding dims
// 4 l .. 4 l + 3.  Merges the cache partials of the query and the draft keys it may see.
__global__ __launch_bounds__(256)
void attn_combine_kernel(const int32_t* __restrict__ ctx, int T_max,
                         const uint16_t* __restrict__ Qd, const uint16_t* __restrict__ Kd,
                         const uint16_t* __restrict__ Vd, const int32_t* __restrict__ parent,
                         int Hkv, int G, int N, int rows, int nsplit,
                         const float* __restrict__ work, float* __restrict__ O,
                         int32_t* __restrict__ status)
{
    const int lane = threadIdx.x & 63;
    const int bk = blockIdx.y;
    const int b = bk / Hkv;
    const int kvh = bk - b * Hkv;
    const int Hq = Hkv * G;
    const int Nq = N * G;
    const int craw = ctx[b];
    const int c = clamp_ctx(craw, T_max);
    if (threadIdx.x == 0 && blockIdx.x == 0 && kvh == 0 && craw != c) report(status, TREEWY_ECTX);
    const int qi = 4 * blockIdx.x + (threadIdx.x >> 6);
    if (qi >= Nq) return;                       // the whole wave
    const int t = qi / G;
    const int hq = kvh * G + (qi - t * G);
    const int nqb = (Nq + kQB - 1) / kQB;
    const int qq = qi % kQB;
    const int used = (c + rows - 1) / rows;
    const float* base = work + static_cast<size_t>(bk * nqb + qi / kQB) * nsplit * kPartFloats;
    const int d0 = 4 * lane;

    // Everything that does not depend on the tree is requested first: the query slice, the
    // tree, and the cache partials' maxima and sums (lane s: split s, first 64 splits).
    const uint16_t* qrow = Qd + (static_cast<size_t>(b * N + t) * Hq + hq) * DA + d0;
    float q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = bf16_to_f32(qrow[e]);
    int pj = lane < N ? parent[b * N + lane] : -1;
    float ms = -INFINITY, ls = 0.f;
    if (lane < used) {
        ms = base[static_cast<size_t>(lane) * kPartFloats + kQB * DA + qq];
        ls = base[static_cast<size_t>(lane) * kPartFloats + kQB * DA + kQB + qq];
    }

    // the ancestors-or-self of t from the whole tree at once (lane = node, pointer jumping; a
    // malformed parent ends the path there and is reported)
    const bool badl = lane < N && (pj < -1 || pj >= lane);
    if (badl) pj = -1;
    uint64_t am = lane < N ? (1ull << lane) : 0ull;
    int bad = badl ? 1 : 0;
    for (int r = 0; (1 << r) < N; ++r) {        // depth <= N: ceil(log2 N) rounds
        const int src = pj < 0 ? lane : pj;
        const uint32_t lo = __shfl(static_cast<uint32_t>(am), src);
        const uint32_t hi = __shfl(static_cast<uint32_t>(am >> 32), src);
        const int bj = __shfl(bad, src);
        const int jj = __shfl(pj, src);
        if (pj >= 0) { am |= (static_cast<uint64_t>(hi) << 32) | lo; bad |= bj; pj = jj; }
    }
    const uint32_t anc_lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(am), t));
    const uint32_t anc_hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(am >> 32), t));
    const uint64_t anc = (static_cast<uint64_t>(anc_hi) << 32) | anc_lo;   // no sign extension
    if (__builtin_amdgcn_readlane(bad, t) && lane == 0) report(status, TREEWY_ETREE);
    const int na = __popcll(anc);               // 1 .. 64

    const float sscale = kLog2e / 16.0f;
    const uint16_t* Kh = Kd + static_cast<size_t>(kvh) * DA + d0;   // + (b N + n) Hkv DA
    const uint16_t* Vh = Vd + static_cast<size_t>(kvh) * DA + d0;
    const size_t nstride = static_cast<size_t>(Hkv) * DA;
    auto next4 = [&](uint64_t& mm, int (&n4)[4]) {   // the next four ancestors (repeats past the end)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            n4[u] = mm ? __builtin_ctzll(mm) : n4[0];
            if (mm) mm &= mm - 1ull;
        }
    };
    // the first four ancestors' key and value rows go out now, with the cache partials below
    uint64_t mk = anc, mv = anc;
    int nk[4], nv[4];
    next4(mk, nk);
    uint2 kw[4], vw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        kw[u] = *reinterpret_cast<const uint2*>(Kh + (static_cast<size_t>(b) * N + nk[u]) * nstride);
        vw[u] = *reinterpret_cast<const uint2*>(Vh + (static_cast<size_t>(b) * N + nk[u]) * nstride);
    }

    // the cache part relative to its own maximum mc: O_c = sum_s 2^(m_s - mc) O_s,
    // l_c = sum_s 2^(m_s - mc) l_s; 8 rows in flight per lane
    float mc = ms;
    for (int s = lane + 64; s < used; s += 64) mc = fmaxf(mc, base[static_cast<size_t>(s) * kPartFloats + kQB * DA + qq]);
    mc = wave_max(mc);                          // -inf when nothing is cached
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    for (int s0 = 0; s0 < used; s0 += 64) {
        const int s = s0 + lane;
        float w = 0.f;
        if (s < used) {
            const float* ps = base + static_cast<size_t>(s) * kPartFloats;
            const float m_s = s0 == 0 ? ms : ps[kQB * DA + qq];
            const float l_s = s0 == 0 ? ls : ps[kQB * DA + kQB + qq];
            w = __builtin_amdgcn_exp2f(m_s - mc);
            lsum += w * l_s;
        }
        const int n = used - s0 < 64 ? used - s0 : 64;
        int j = 0;
        for (; j + 8 <= n; j += 8) {
            f32x4_t x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                x[u] = *reinterpret_cast<const f32x4_t*>(
                    base + static_cast<size_t>(s0 + j + u) * kPartFloats + qq * DA + d0);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float wu = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j + u));
                acc += wu * x[u];
            }
        }
        for (; j < n; ++j) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(
                base + static_cast<size_t>(s0 + j) * kPartFloats + qq * DA + d0);
            const float wu = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
            acc += wu * x;
        }
    }

    // scores of the draft keys (four rows at a time); lane j keeps the j-th one
    float sc = -INFINITY;
    for (int j0 = 0; j0 < na; j0 += 4) {
        if (j0 > 0) {
            next4(mk, nk);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                kw[u] = *reinterpret_cast<const uint2*>(Kh + (static_cast<size_t>(b) * N + nk[u]) * nstride);
        }
        float dot[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            dot[u] = q[0] * __uint_as_float(kw[u].x << 16) + q[1] * __uint_as_float(kw[u].x & 0xffff0000u) +
                     q[2] * __uint_as_float(kw[u].y << 16) + q[3] * __uint_as_float(kw[u].y & 0xffff0000u);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1)
#pragma unroll
            for (int u = 0; u < 4; ++u) dot[u] += __shfl_xor(dot[u], o);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (lane == j0 + u && j0 + u < na) sc = dot[u] * sscale;
    }

    // the overall maximum; the cache part rescaled to it, then the draft terms
    const float mt = fmaxf(mc, wave_max(sc));   // finite: the node sees itself
    const float rc = used > 0 ? __builtin_amdgcn_exp2f(mc - mt) : 0.f;
    acc *= rc;
    const float wd = lane < na ? __builtin_amdgcn_exp2f(sc - mt) : 0.f;
    lsum = lsum * rc + wd;
    lsum = wave_sum(lsum);
    for (int j0 = 0; j0 < na; j0 += 4) {
        if (j0 > 0) {
            next4(mv, nv);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                vw[u] = *reinterpret_cast<const uint2*>(Vh + (static_cast<size_t>(b) * N + nv[u]) * nstride);
        } else {
            next4(mv, nv);                      // the first four rows are already here
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float w = j0 + u < na ? __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wd), j0 + u)) : 0.f;
            acc[0] += w * __uint_as_float(vw[u].x << 16);
            acc[1] += w * __uint_as_float(vw[u].x & 0xffff0000u);
            acc[2] += w * __uint_as_float(vw[u].y << 16);
            acc[3] += w * __uint_as_float(vw[u].y & 0xffff0000u);
        }
    }
    const float inv = 1.0f / lsum;
    float* orow = O + (static_cast<size_t>(b * N + t) * Hq + hq) * DA + d0;
    *reinterpret_cast<f32x4_t*>(orow) = acc * inv;
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


// Cache rows per split for a launch: about kTargetBlocks workgroups over the (sequence, key/value
// head, query block) triples, whole tiles, at least kMinSplit rows.
int split_rows(int B, int Hkv, int G, int N, int T_max) {
    const long long pairs = static_cast<long long>(B) * Hkv * ((static_cast<long long>(N) * G + kQB - 1) / kQB);
    const long long want = (kTargetBlocks + pairs - 1) / pairs;
    long long rows = (T_max + want - 1) / want;
    rows = (rows + kTile - 1) / kTile * kTile;
    return static_cast<int>(rows < kMinSplit ? kMinSplit : rows);
}

int split_count(int T_max, int rows) { return (T_max + rows - 1) / rows; }

}  // namespace

size_t attention_workspace_bytes(int B, int Hkv, int G, int N, int T_max) {
    const size_t nsplit = split_count(T_max, split_rows(B, Hkv, G, N, T_max));
    const size_t nqb = (static_cast<size_t>(N) * G + kQB - 1) / kQB;
    return static_cast<size_t>(B) * Hkv * nqb * nsplit * kPartFloats * sizeof(float);
}

hipError_t launch_tree_attention(const AttentionArgs& a, hipStream_t stream) {
    const int rows = split_rows(a.B, a.Hkv, a.G, a.N, a.T_max);
    const int nsplit = split_count(a.T_max, rows);
    const int nqb = (a.N * a.G + kQB - 1) / kQB;
    hipLaunchKernelGGL(attn_partial_kernel, dim3(nsplit, nqb, a.B * a.Hkv), dim3(128), 0, stream,
                       static_cast<const uint16_t*>(a.Kc), static_cast<const uint16_t*>(a.Vc),
                       a.ctx, a.T_max, static_cast<const uint16_t*>(a.Qd), a.Hkv, a.G, a.N, rows,
                       static_cast<float*>(a.work));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((a.N * a.G + 3) / 4, a.B * a.Hkv), dim3(256), 0,
                       stream, a.ctx, a.T_max, static_cast<const uint16_t*>(a.Qd),
                       static_cast<const uint16_t*>(a.Kd), static_cast<const uint16_t*>(a.Vd),
                       a.parent, a.Hkv, a.G, a.N, rows, nsplit, static_cast<const float*>(a.work),
                       a.O, a.status);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// The fixed device array of treewy_tree_attention_noalloc: the split partials of a launch
// go here instead of a caller's workspace.  Each GPU the library runs on holds its own copy
// for the life of the process.  In host code `scratch` names a host-side stand-in, not a
// device address: its address on the current device is resolved once per device with
// hipGetSymbolAddress and only that address is passed to the kernels.

static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

namespace {

std::atomic<void*> g_scratch_addr[64];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on the first call on a device, with
// that device current).
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

hipError_t launch_tree_attention_noalloc(const AttentionArgs& a, hipStream_t stream) {
    // the caller has checked that the partials fit (attention_workspace_bytes <= the array)
    void* p = nullptr;
    hipError_t e = scratch_address(&p);
    if (e != hipSuccess) return e;
    AttentionArgs b = a;
    b.work = p;
    return launch_tree_attention(b, stream);
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
