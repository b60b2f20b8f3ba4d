// TreeWY tree verification on gfx950.
//
// Paper: "TreeWY: Speculative Verification for Gated DeltaNet Hybrids" (arXiv 2608.20961),
// §3 "Verifying a draft", Eq. (2), and the per-node readout o_t = S_t q_t with S_t written
// through the unrolled form of §3 "Reconstruct on commit" (Eq. 3 evaluated at a = t).
//
// Every kernel here computes, per (sequence, head):
//   1. tree bookkeeping: ancestor masks, depths, cumulative gates g_t (pointer jumping);
//   2. P[t] = S0 k_t and Y[t] = S0 q_t, S0 read once from HBM;
//   3. R[t] = b_t (v_t - g_t P[t]); coefficients on ancestor pairs only:
//      C = b_t (g_t/g_i)(k_t . k_i) for strict ancestors, W = (g_t/g_i)(k_i . q_t);
//   4. forward substitution U[t] = R[t] - sum_i C[t,i] U[i], ancestors before descendants
//      (value rows are independent);
//   5. readout O[t] = g_t Y[t] + sum_{i anc-or-self} W[t,i] U[i]; O, U, gamma written once;
// and, in the fused forms, the previous step's commit (Eq. 3) on the state first.
// Kernels: fp32 inputs (verify_f32_kernel); bf16 inputs on trees of up to 16 nodes
// (verify_small_kernel), the plain verify on 17 to 32 nodes (verify_large_kernel), and one
// head per item for the rest: the fused and deferred steps on 17 to 64 nodes, the plain
// verify on 33 to 64 (verify_head_kernel).

#include "device_common.h"
#include "launch.h"

#include <atomic>

namespace treewy {

namespace {

// ---------------------------------------------------------------------------------------
// bf16 inputs: the S0 contractions on the matrix cores.
//
// P^T = S0 [K;Q]^T is a [128 x 128] x [128 x 2N] product per head.  S0 is fp32; it is split
// as S0 = hi + lo, hi = S0 rounded to bf16 and lo = the (exact) remainder rounded to bf16,
// so |S0 - hi - lo| <= 2^-18 |S0|.  q and k are exact in bf16, so two bf16 MFMAs with fp32
// accumulation give an fp32-grade product.
//
// S0 goes HBM -> LDS directly (global_load_lds_dwordx4: lane l of a wave instruction lands
// at base + 16 l), fully coalesced: a wave instruction covers two whole rows.  Within a row
// the 16-byte chunk c is stored at slot c ^ (row % 16), which makes the MFMA operand reads
// below conflict-free.  Operands follow v_mfma_f32_16x16x32_bf16: lane L holds row L % 16
// of a 16-row tile and 8 consecutive k's from 8 (L / 16); both operands use the same k
// order, so the sums are those of the plain product.  The same key fragments give the Gram
// matrix K [K;Q]^T (k_m.k_n and k_m.q_n), whose ancestor entries are the solve coefficients.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ void split_hi_lo(f32x4_t a, f32x4_t b, bf16x8_t& hi, bf16x8_t& lo) {
    const f32x8_t f = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    hi = __builtin_convertvector(f, bf16x8_t);                       // round to nearest even
    const u32x4_t hw = __builtin_bit_cast(u32x4_t, hi);
    f32x8_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[2 * j] = f[2 * j] - __uint_as_float(hw[j] << 16);          // exact remainders
        r[2 * j + 1] = f[2 * j + 1] - __uint_as_float(hw[j] & 0xffff0000u);
    }
    lo = __builtin_convertvector(r, bf16x8_t);
}

// ---------------------------------------------------------------------------------------
// Small trees (N <= 16): persistent workgroups of 256 lanes over (head, value-row half)
// items, the solve in registers.
//
// Every input of an item reaches LDS by direct HBM -> LDS transfers (global_load_lds), with
// no trip through registers: the item's 64 S0 rows (32 KB), its keys and queries (2N rows of
// 256 B), the item's half of its values (N rows of 128 B) and the parents and gates (one
// 4-byte gather).  A workgroup reads its item's operands out of LDS into registers, and at
// once the next item's transfers are issued into the same buffers, so the next item streams
// in while the current one is solved and written.  The four waves fetch the keys and queries
// once per workgroup instead of once per wave.  The two halves of a head go to workgroups on
// the same XCD (slots s and s + 8 of every 16) in the same round, so the head's keys and
// queries are fetched into that XCD's L2 once.
//
// The contractions run on the matrix cores, on this half's 64 rows: wave w owns rows
// 16w..16w+15.  Keys occupy output columns 0..N-1 of tile 0 and queries columns N..2N-1
// (tile 0 or 1), so after the contractions lane L of a wave holds P[t][v..v+3] for node
// t = L % 16 and rows v = 16w + 4 (L / 16) .. +3.  The forward substitution and the readout
// then run on those registers: every lane walks its node's ancestors root first (the set
// bits of its ancestor mask, in increasing order = increasing depth), fetching the
// ancestor's U from the lane that holds it (same 16-lane group) with a lane permute.  At
// step d every node at depth > d subtracts the term of its depth-d ancestor, whose value
// became final at step d - 1, so nodes of all depths advance together and the number of
// steps is the tree depth.  Coefficients come from the Gram matrix staged in LDS.

constexpr int kSmallThreads = 256;
// s_waitcnt operand (gfx9 encoding): vmcnt = 2 (bits 3:0 and 15:14), expcnt and lgkmcnt
// left at their maxima (no wait on them)
constexpr int kWaitAllButTwoStores = 2 | (7 << 4) | (15 << 8);
constexpr int kWaitAllButEight = 8 | (7 << 4) | (15 << 8);
constexpr int kWaitLdsOnly = 0xC07F;            // LDS/scalar count 0, the rest left free
// dword 3 of a raw (unstrided, range-checked) buffer descriptor on gfx9-family parts
constexpr int kRawBufferFlags = 0x00020000;
// buffer-store cache policy: non-temporal (O and U of the fused kernel on 9-16 nodes; on up
// to 8 nodes the default policy measured faster)
constexpr int kStreamAux = 2;
constexpr int kSmallRows = 64;              // value rows per item
constexpr int kSmallParts = D / kSmallRows; // items per head

// LDS of one small-tree workgroup, as byte offsets sized for the tree at hand (N nodes,
// NCT column tiles), so that small trees leave room for more resident workgroups.  After the
// S0 rows [64][128] fp32: keys in rows 0 .. 4 ceil(N/4) - 1 of the key/query area and queries
// right after them (bf16 rows of 256 B); the item's half of the values (rows of 128 B);
// parents, alphas, betas (words 0-15, 16-31, 32-47) and one more word (48); the Gram matrix
// [16][16 NCT] fp32.  With the fused commit: `path` U_prev half-rows (256 B) and K_prev rows
// (256 B), the path's gammas [64] and the previous tree's parents [64].  With the deferred
// commit also: the sequence's log length (one word, repeated), the head's log scale (one
// word, repeated), and the log's Lmax u-half-rows (256 B) and key rows (256 B).  16-byte
// chunk c of a row r of S0 or of the key/query area is stored at chunk c ^ (r % 16), which
// keeps the MFMA operand reads free of bank conflicts.
struct SmallLds {
    uint32_t kq, v, sm, g, pu, pk, pg, idx, il, lg, lu, lk, bytes;
    uint32_t set;                               // second input set at +set (0: one set)
    int path;                                   // path rows staged per chunk (fused)
};

// The fused kernel on trees of up to 8 nodes keeps two sets of per-item inputs (key/query and
// value rows, parents/gates, path rows, previous tree): the next item's set is requested at
// the top of this item, and the next item's S rows as soon as each wave has taken its own
// rows into registers, so both stream in during this item's solve.
__host__ __device__ constexpr bool small_two_sets(int nct, int mode) { return nct == 1 && mode == 1; }

// mode: 0 plain verify, 1 fused commit, 2 deferred commit (log of lmax terms)
__host__ __device__ inline SmallLds small_lds(int N, int nct, int mode, int lmax = 0) {
    SmallLds L;
    L.path = N <= 4 ? 4 : 8;
    if (small_two_sets(nct, mode)) {
        // S rows, the Gram matrix, then two sets of [key/query rows, values, parents/gates,
        // path rows, path gammas, previous tree]
        L.g = kSmallRows * D * 4;
        const uint32_t s0 = L.g + 1024u * static_cast<uint32_t>(nct);
        L.kq = s0;
        L.v = L.kq + 2048u * static_cast<uint32_t>((N + 3) / 4);
        L.sm = L.v + 1024u * static_cast<uint32_t>((N + 7) / 8);
        L.pu = L.sm + 256u;
        L.pk = L.pu + 256u * L.path;
        L.pg = L.pk + 256u * L.path;
        L.idx = L.pg + 256u;
        L.il = L.lg = L.lu = L.lk = L.idx + 256u;   // no log
        L.set = L.idx + 256u - s0;
        L.bytes = L.idx + 256u + L.set;
        return L;
    }
    L.set = 0;
    L.kq = kSmallRows * D * 4;
    L.v = L.kq + 2048u * static_cast<uint32_t>((N + 3) / 4);
    L.sm = L.v + 1024u * static_cast<uint32_t>((N + 7) / 8);
    L.g = L.sm + 256u;
    const uint32_t end = L.g + 1024u * static_cast<uint32_t>(nct);
    L.pu = end;
    L.pk = L.pu + 256u * L.path;
    L.pg = L.pk + 256u * L.path;
    L.idx = L.pg + 256u;
    L.il = L.idx + 256u;
    L.lg = L.il + 256u;
    // the log rows arrive four to a transfer: room for a multiple of four
    const uint32_t lrows = 4u * static_cast<uint32_t>((lmax + 3) / 4);
    L.lu = L.lg + 256u;
    L.lk = L.lu + 256u * lrows;
    L.bytes = mode == 0 ? end : mode == 1 ? L.idx + 256u : L.lk + 256u * lrows;
    return L;
}

// Waves per SIMD the registers are budgeted for (= resident workgroups per CU): four for the
// plain kernel on trees of up to 8 nodes; three where LDS allows no more (16 nodes) or the
// fused commit needs the registers; two for the deferred commit on 16-node trees, whose LDS
// (with a log of 16 terms) leaves room for two.
template <int NCT, int MODE>
constexpr int kSmallWavesPerSimd = (NCT == 2 && MODE == 2) ? 2 : (NCT == 2 || MODE != 0) ? 3 : 4;

// resident workgroups per CU: the register budget, within the 160 KB of LDS
inline int small_wgs(uint32_t bytes, int regs_wgs) {
    const uint32_t w = (160u * 1024u) / bytes;
    return w > static_cast<uint32_t>(regs_wgs) ? regs_wgs : static_cast<int>(w);
}

// Item number -> (head, half).  Slots s and s + 8 of every group of 16 run on one XCD and
// take the two halves of one head; a grid that is not a multiple of 16 uses plain order.
__device__ __forceinline__ void small_item(int round, int slot, int grid, int& bh, int& part) {
    int item;
    if ((grid & 15) == 0) {
        const int pair = (grid >> 1) * round + ((slot >> 4) << 3) + (slot & 7);
        item = 2 * pair + ((slot >> 3) & 1);
    } else {
        item = grid * round + slot;
    }
    bh = item >> 1;
    part = item & 1;
}

// Eight HBM -> LDS row-pair loads (global_load_lds_dwordx4) of one wave: load i sends lane
// l's 16 bytes from base + voff[i] to LDS byte lds0 + 1024 i + 16 l.  Written as one asm block
// so the compiler does not treat every later LDS access as a possible alias of the transfer
// (it would wait for it right away); the caller waits on vmcnt before reading the rows.
// M0 holds the LDS destination and is restored afterwards; only vector memory is accessed.
// With NT the loads carry the non-temporal (streaming) hint: for state rows that are read
// once and then overwritten, so they are not kept in the caches at the expense of other data.
#define TREEWY_ROWS_X8(POL)                                                                    \
    "s_mov_b32 %0, m0\n\t"                                                                   \
    "s_mov_b32 m0, %1\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %9, %17" POL "\n\t"      \
    "s_mov_b32 m0, %2\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %10, %17" POL "\n\t"     \
    "s_mov_b32 m0, %3\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %11, %17" POL "\n\t"     \
    "s_mov_b32 m0, %4\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %12, %17" POL "\n\t"     \
    "s_mov_b32 m0, %5\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %13, %17" POL "\n\t"     \
    "s_mov_b32 m0, %6\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %14, %17" POL "\n\t"     \
    "s_mov_b32 m0, %7\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %15, %17" POL "\n\t"     \
    "s_mov_b32 m0, %8\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %16, %17" POL "\n\t"     \
    "s_mov_b32 m0, %0"

template <bool NT>
__device__ __forceinline__ void dma_rows_x8(const void* base, const uint32_t (&voff)[8],
                                            uint32_t lds0) {
    uint32_t save;
#define TREEWY_ROWS_X8_OPERANDS                                                                 \
        : "=&s"(save)                                                                           \
        : "s"(lds0), "s"(lds0 + 1024u), "s"(lds0 + 2048u), "s"(lds0 + 3072u),                   \
          "s"(lds0 + 4096u), "s"(lds0 + 5120u), "s"(lds0 + 6144u), "s"(lds0 + 7168u),           \
          "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "v"(voff[5]),   \
          "v"(voff[6]), "v"(voff[7]), "s"(base)                                                 \
        : "memory"
    if constexpr (NT)
        asm volatile(TREEWY_ROWS_X8(" nt") TREEWY_ROWS_X8_OPERANDS);
    else
        asm volatile(TREEWY_ROWS_X8("") TREEWY_ROWS_X8_OPERANDS);
#undef TREEWY_ROWS_X8_OPERANDS
}
#undef TREEWY_ROWS_X8

// Two HBM -> LDS loads of 16 bytes per lane: lane l's bytes from base + voff0 land at LDS
// byte lds0 + 16 l, those from base + voff1 at lds0 + 1024 + 16 l.  lds0 and base are
// wave-uniform.
template <bool NT>
__device__ __forceinline__ void dma_rows_x2(const void* base, uint32_t voff0, uint32_t voff1,
                                            uint32_t lds0) {
    uint32_t save;
    if constexpr (NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %3, %5 nt\n\t"
            "s_mov_b32 m0, %2\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %4, %5 nt\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(save)
            : "s"(lds0), "s"(lds0 + 1024u), "v"(voff0), "v"(voff1), "s"(base)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %3, %5\n\t"
            "s_mov_b32 m0, %2\n\t" "s_nop 0\n\t" "global_load_lds_dwordx4 %4, %5\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(save)
            : "s"(lds0), "s"(lds0 + 1024u), "v"(voff0), "v"(voff1), "s"(base)
            : "memory");
}

// A pointer that is the same in every lane, kept in scalar registers (the compiler cannot
// always prove it uniform).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t x = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One HBM -> LDS load of 16 bytes per lane: lane l's bytes from base + voff land at LDS byte
// lds + 16 l.
__device__ __forceinline__ void dma_x4(const void* base, uint32_t voff, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);      // wave-uniform by construction
    base = uniform_ptr(base);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(base)
        : "memory");
}

// One HBM -> LDS gather of 4 bytes per lane: lane l's word at its own address lands at LDS
// byte lds + 4 l.
__device__ __forceinline__ void dma_gather_x1(const void* addr, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);      // wave-uniform by construction
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(addr)
        : "memory");
}

// One HBM -> LDS gather of 16 bytes per lane: lane l's bytes at its own address land at LDS
// byte lds + 16 l.
__device__ __forceinline__ void dma_gather_x4(const void* addr, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);      // wave-uniform by construction
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(addr)
        : "memory");
}

// One HBM -> LDS load of 4 bytes per lane: lane l's word at base + voff lands at LDS byte
// lds + 4 l.
__device__ __forceinline__ void dma_x1(const void* base, uint32_t voff, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);      // wave-uniform by construction
    base = uniform_ptr(base);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(base)
        : "memory");
}

// S0 rows of an item -> LDS: wave w takes rows 16w..16w+15, two whole rows per wave load;
// chunk c of row r lands at slot c ^ (r % 16).  `wave` is wave-uniform (an SGPR), so the
// LDS destinations are scalar; the source is a scalar base plus a 32-bit lane offset.
template <bool NT>
__device__ __forceinline__ void small_issue_s0(const float* S0, float* buf, int bh, int part,
                                               int wave, int lane) {
    const char* src = reinterpret_cast<const char*>(S0) +
                      (static_cast<size_t>(bh) * D + part * kSmallRows) * D * sizeof(float);
    const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
    const uint32_t slot = static_cast<uint32_t>(lane) & 31u;
    uint32_t voff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t r = 16u * wave + 2u * i + hl;
        voff[i] = r * (D * 4u) + 16u * (slot ^ ((2u * i + hl) & 15u));
    }
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf + 16 * wave * D));
    dma_rows_x8<NT>(src, voff, lds0);
}

// Part of an item's S rows -> LDS, in the layout of small_issue_s0: wave w's row pairs
// i0 .. i0 + 2 n - 1 (pair i: rows 16w + 2i and 16w + 2i + 1, one whole row per half-wave),
// two pairs per dma_rows_x2.  The kernels that request their next item's rows during the
// current one split the request into such parts, spread over the item: issued at once, the
// eight transfers of a wave stall its issue (the CU's queue of vector-memory requests is
// full) while the other phases wait for it; in parts they queue behind work that does not.
template <bool NT>
__device__ __forceinline__ void issue_s_pairs(const float* S0, uint32_t lds_addr, int bh, int part,
                                              int i0, int n, int wave, int lane) {
    const void* src = uniform_ptr(reinterpret_cast<const char*>(S0) +
                                  (static_cast<size_t>(bh) * D + part * kSmallRows) * D *
                                      sizeof(float));
    const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
    const uint32_t slot = static_cast<uint32_t>(lane) & 31u;
    for (int j = 0; j < n; ++j) {
        const uint32_t i = static_cast<uint32_t>(i0 + 2 * j);
        const uint32_t r0 = 16u * wave + 2u * i + hl;
        const uint32_t voff0 = r0 * (D * 4u) + 16u * (slot ^ ((2u * i + hl) & 15u));
        const uint32_t voff1 = (r0 + 2u) * (D * 4u) + 16u * (slot ^ ((2u * i + 2u + hl) & 15u));
        const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
            lds_addr + 16u * static_cast<uint32_t>(wave) * D * 4u + 1024u * i);
        dma_rows_x2<NT>(src, voff0, voff1, lds0);
    }
}

// The rest of an item's inputs -> LDS, as a list of whole-wave transfers dealt round-robin
// to the four waves: ceil(N/4) loads of four key rows, as many of four query rows,
// ceil(N/8) loads of eight value half-rows, and one gather of parent, alpha and beta (lanes
// 0-15, 16-31, 32-47) plus the word at `extra` (lanes 48-63; their own parent again when it
// is null).  Lanes past the last node load node 0 again, into rows nobody reads.
__device__ __forceinline__ void small_issue_inputs(const uint16_t* Q, const uint16_t* K,
                                                   const uint16_t* V, const float* alpha,
                                                   const float* beta, const int32_t* parent,
                                                   int H, int N, int bh, int part, int wave,
                                                   int lane, uint32_t lds, const SmallLds& L,
                                                   const int32_t* extra) {
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;
    const uint32_t row_bytes = static_cast<uint32_t>(H) * D * 2;   // between nodes of a head
    const uint16_t* Kh = K + (node0 * H + h) * D;
    const uint16_t* Qh = Q + (node0 * H + h) * D;
    const uint16_t* Vh = V + (node0 * H + h) * D + part * kSmallRows;
    const uint32_t un = static_cast<uint32_t>(N);
    const int nq4 = (N + 3) >> 2;
    const int nv8 = (N + 7) >> 3;
    const int jobs = 2 * nq4 + nv8 + 1;
    for (int j = wave; j < jobs; j += 4) {
        if (j < 2 * nq4) {
            const bool is_q = j >= nq4;
            const uint32_t lr = static_cast<uint32_t>(lane) >> 4;
            const uint32_t r = 4u * j + lr;                           // LDS row
            const uint32_t n = 4u * (is_q ? j - nq4 : j) + lr;        // node
            const uint32_t c = (static_cast<uint32_t>(lane) & 15u) ^ (r & 15u);
            dma_x4(is_q ? Qh : Kh, (n < un ? n : 0u) * row_bytes + 16u * c,
                   lds + L.kq + 1024u * j);
        } else if (j < 2 * nq4 + nv8) {
            const int jv = j - 2 * nq4;
            const uint32_t n = 8u * jv + (static_cast<uint32_t>(lane) >> 3);
            const uint32_t c = static_cast<uint32_t>(lane) & 7u;
            dma_x4(Vh, (n < un ? n : 0u) * row_bytes + 16u * c, lds + L.v + 1024u * jv);
        } else {
            const uint32_t t = static_cast<uint32_t>(lane) & 15u;
            const uint32_t kind = static_cast<uint32_t>(lane) >> 4;
            const size_t n = node0 + (t < un ? t : 0u);
            const void* src = kind == 1 ? static_cast<const void*>(alpha + n * H + h)
                            : kind == 2 ? static_cast<const void*>(beta + n * H + h)
                            : kind == 3 && extra ? static_cast<const void*>(extra)
                                                 : static_cast<const void*>(parent + n);
            dma_gather_x1(src, lds + L.sm);
        }
    }
}

// ---------------------------------------------------------------------------------------
// The previous step's commit fused into this step's verify (paper §3 "Reconstruct on
// commit", Eq. 3, applied to S0 on its way into the contractions).
//
// S holds the state before the previous step's commit.  For each item the S rows arrive in
// LDS as above; each lane takes its 32 values of row r into registers, replaces them by
//   S_a[r][k] = g_a S[r][k] + sum over i on the path of a of (g_a / g_i) U_prev[i][r] k_i[k]
// (a = the previous step's accepted node; nothing when a = -1), writes them back to S and
// splits them into the bf16 operands of this step's contractions.  So the state is read once
// and written once per step, and the commit costs no launch of its own.
//
// The path's rows (U_prev half-rows, K_prev rows, gammas) must be in flight with the item's
// other transfers, so the path has to be known one item early; it comes from the previous
// tree and accepted node of the item's sequence, which are fetched two items early (the
// parents into an LDS index slot, the accepted node as the spare word of the input gather).
// At the top of item i the workgroup derives the path of item i + 1 (pointer jumping over
// the previous tree, lane = node); at the refill point of item i the first rows of that path
// (4 for trees of up to 4 nodes, else 8) go out together with item i + 1's S rows, and the
// index of item i + 2 is fetched.  A longer path is finished in further chunks with a
// blocking wait.

struct CommitIn {
    float* S;                               // state, updated in place
    const float* U;                         // U of the previous step [B][Np][H][128]
    const uint16_t* K;                      // its keys, bf16 [B][Np][H][128]
    const float* gamma;                     // its cumulative gates [B][Np][H]
    const int32_t* parent;                  // its tree [B][Np]
    const int32_t* accepted;                // its accepted node [B], -1 = none
    int Np;                                 // its node count
    int short_path;                         // 17-64 nodes, fused commit: paths up to this
                                            // long (0 or 8) go on the vector ALUs (set at
                                            // launch)
};

// The deferred commit's log of one step (see the kernel below): per (sequence, head) up to
// Lmax rank-one terms u~_j k_j^T and a scale, such that the committed state is
// scale * (S + sum_j u~_j k_j^T).  Header words are read from *_in and written to *_out.
struct DeferLog {
    float* U;                               // [B][H][Lmax][128] fp32 terms u~
    uint16_t* K;                            // [B][H][Lmax][128] bf16 keys
    const float* scale_in;                  // [B][H]
    float* scale_out;
    const int32_t* len_in;                  // [B] terms in use (every head of a sequence alike)
    int32_t* len_out;
    int Lmax;
};

// One item's commit: the path of the accepted node as a mask, its length, and in lane q the
// q-th path node in increasing order (root first).
struct PathInfo {
    uint64_t mask;
    int depth;                              // 0: nothing to commit
    int pn;
};

// Sequence b's previous tree -> the LDS index slot (lane n: parent of node n; lanes past Np
// repeat node 0).
__device__ __forceinline__ void fused_issue_index(const CommitIn& c, int b, int lane,
                                                  uint32_t slot) {
    const int n = lane < c.Np ? lane : 0;
    dma_gather_x1(c.parent + static_cast<size_t>(b) * c.Np + n, slot);
}

// The path of accepted node `a`, by every wave (lane = node of the previous tree, p_raw = its
// parent, -1 past Np): pointer jumping gives each node its inclusive ancestor mask and whether
// a malformed parent lies on its way up.  An accepted node outside [-1, Np - 1] or a malformed
// path leaves nothing to commit and is reported when `reporter` is set.
__device__ __forceinline__ PathInfo fused_path(int p_raw, int a, int Np, int lane,
                                               bool reporter, int32_t* status) {
    a = __builtin_amdgcn_readfirstlane(a);
    const bool bad = lane < Np && (p_raw < -1 || p_raw >= lane);
    int j = bad ? -1 : p_raw;
    uint64_t am = lane < Np ? (1ull << lane) : 0ull;
    int badp = bad ? 1 : 0;
    // a node's depth is at most Np (parents precede their children): ceil(log2 Np) rounds
    for (int r = 0; (1 << r) < Np; ++r) {
        const int src = j < 0 ? lane : j;
        const uint64_t aj = shfl_u64(am, src);
        const int bj = __shfl(badp, src);
        const int jj = __shfl(j, src);
        if (j >= 0) { am |= aj; badp |= bj; j = jj; }
    }
    PathInfo pi;
    pi.mask = 0ull;
    pi.depth = 0;
    pi.pn = 0;
    if (a < -1 || a >= Np) {
        if (reporter && lane == 0) report(status, TREEWY_EACCEPT);
        return pi;
    }
    if (a < 0) return pi;
    const uint64_t m = shfl_u64(am, a);
    const int mbad = __shfl(badp, a);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(m));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(m >> 32));
    if (__builtin_amdgcn_readfirstlane(mbad)) {
        if (reporter && lane == 0) report(status, TREEWY_ETREE);
        return pi;
    }
    uint64_t mm = (static_cast<uint64_t>(hi) << 32) | lo;
    pi.mask = mm;
    pi.depth = __popcll(mm);
    for (int q = 0; mm != 0ull; ++q) {
        const int n = __builtin_ctzll(mm);
        mm &= mm - 1ull;
        if (lane == q) pi.pn = n;
    }
    return pi;
}

// Path rows P c .. P c + P - 1 (P = L.path) of an item -> LDS: U_prev half-rows (this item's
// 64 value rows) and K_prev rows, four per transfer, and with the first chunk the gammas of
// the whole path (one gather).  Slots past the path repeat its first node.
__device__ __forceinline__ void fused_issue_path(const CommitIn& c, const PathInfo& pi, int chunk,
                                                 int bh, int part, int H, int wave, int lane,
                                                 uint32_t lds, const SmallLds& L) {
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * c.Np;
    const int P = L.path;
    const int cnt = pi.depth - P * chunk < P ? pi.depth - P * chunk : P;
    const int nj = (cnt + 3) >> 2;
    const int jobs = 2 * nj + (chunk == 0 ? 1 : 0);
    const float* Uh = c.U + (node0 * H + h) * D + part * kSmallRows;
    const uint16_t* Kh = c.K + (node0 * H + h) * D;
    const uint32_t col16 = 16u * (static_cast<uint32_t>(lane) & 15u);
    for (int j = wave; j < jobs; j += 4) {
        if (j < 2 * nj) {
            const bool is_k = j >= nj;
            const int jj = is_k ? j - nj : j;
            const int q = 4 * jj + (lane >> 4);
            const uint32_t n = static_cast<uint32_t>(__shfl(pi.pn, P * chunk + (q < cnt ? q : 0)));
            if (is_k)
                dma_x4(Kh, n * static_cast<uint32_t>(H) * (D * 2u) + col16, lds + L.pk + 1024u * jj);
            else
                dma_x4(Uh, n * static_cast<uint32_t>(H) * (D * 4u) + col16, lds + L.pu + 1024u * jj);
        } else {
            const int n = __shfl(pi.pn, lane < pi.depth ? lane : 0);
            dma_gather_x1(c.gamma + (node0 + n) * H + h, lds + L.pg);
        }
    }
}

// A log length read from memory, kept inside [0, lmax] (the header of a caller who broke the
// contract; TREEWY_ELOG is reported where the length is used).
__device__ __forceinline__ int log_len(int v, int lmax) {
    return v < 0 ? 0 : (v > lmax ? lmax : v);
}

// The first `len` log terms of an item -> LDS (its half of each u~ row, every key row, four
// rows per transfer), and the head's log scale (one word, repeated over 64 words).
__device__ __forceinline__ void defer_issue_log(const DeferLog& dl, int len, int bh, int part,
                                                int wave, int lane, uint32_t lds,
                                                const SmallLds& L) {
    const int nj = (len + 3) >> 2;
    const int jobs = 2 * nj + 1;
    const size_t row0 = static_cast<size_t>(bh) * dl.Lmax;
    const uint32_t col16 = 16u * (static_cast<uint32_t>(lane) & 15u);
    for (int j = wave; j < jobs; j += 4) {
        if (j < 2 * nj) {
            const bool is_k = j >= nj;
            const int jj = is_k ? j - nj : j;
            const int q = 4 * jj + (lane >> 4);
            const uint32_t r = static_cast<uint32_t>(q < len ? q : 0);
            if (is_k)
                dma_x4(dl.K + row0 * D, r * (D * 2u) + col16, lds + L.lk + 1024u * jj);
            else
                dma_x4(dl.U + row0 * D + part * kSmallRows, r * (D * 4u) + col16,
                       lds + L.lu + 1024u * jj);
        } else {
            dma_x1(dl.scale_in + bh, 0u, lds + L.lg);
        }
    }
}

// ---------------------------------------------------------------------------------------
// fp32 inputs: one workgroup of 256 lanes per (sequence, head, block of 16 value rows), so
// that a head's 128 rows run on eight workgroups side by side (rows are independent: row v
// of the state only meets row v of S0 and column v of V, U and O).
//
// Every input of a workgroup reaches LDS in one batch of direct HBM -> LDS transfers issued
// at once: its 16 S0 rows, the head's key and query rows, its 16-row slice of every value
// row, the parents, alphas and betas, and (fused) the previous tree, accepted node and, for
// a previous tree of up to 16 nodes, all its K_prev rows, U_prev slices and gammas.  One
// wave walks the tree (pointer jumping); with the fused commit another derives the accepted
// path.  A larger previous tree has only its path's rows fetched, in a second batch, 16 path
// nodes at a time.  The products P^T = S0 K^T and Y^T = S0 Q^T of the block's rows and the
// Gram tiles K K^T (at and below the diagonal) and K Q^T (at and above it) run on the matrix
// cores with both operands split into bf16 hi + lo (f32_tile), one 16 x 16 tile per wave at
// a time; rows are staged with 16-byte chunk c of row r at c ^ (r % 16), so the operand reads
// are free of bank conflicts.  The forward substitution runs level by level (step d folds in every node's
// depth-d ancestor, final since step d - 1), lanes over (row, node), and the readout sums
// each node's ancestors-or-self.
//
// FUSED: the previous step's commit first (paper §3 "Reconstruct on commit", Eq. 3): the
// 16 rows become g_a S + sum over the accepted path of (g_a / g_i) U_prev[i] k_i^T and are
// written back to S before the contractions, so the fused step is one launch.  The barriers
// order LDS only, so no phase waits for the global stores of an earlier one.

constexpr int kF32Rows = 16;                    // value rows per workgroup
constexpr int kF32Blocks = D / kF32Rows;        // workgroups per head
constexpr int kF32Threads = 256;
constexpr int kF32Waves = kF32Threads / 64;
constexpr int kF32Path = 16;                    // path nodes staged per batch (fused)

struct CommitInF32 {
    float* S;
    const float* U;                             // [B][Np][H][128]
    const float* K;                             // [B][Np][H][128]
    const float* gamma;                         // [B][Np][H]
    const int32_t* parent;                      // [B][Np]
    const int32_t* accepted;                    // [B]
    int Np;
};

// LDS of one fp32 workgroup for N nodes (byte offsets, 16-byte aligned areas): S rows
// [16][128]; key and query rows [N rounded up to 16][128] (whole matrix-core tiles); value
// slices [N rounded up to 16][16]; P, Y, R-then-U [N][16]; k_t . k_i and k_i . q_t [N][N]; the ancestor of t at
// depth j + 1 [N][64] bytes; parents, alphas, betas, previous tree, accepted (64 words each);
// the path rows of one batch: K_prev rows [16][128], U_prev slices [16][16], gammas [64].
struct F32Lds {
    uint32_t s, k, q, v, p, y, u, c, w, at, sm, pk, pu, pg, bytes;
};
__host__ __device__ inline F32Lds f32_lds(int N) {
    F32Lds L;
    const uint32_t n = static_cast<uint32_t>(N);
    const uint32_t n16 = (n + 15u) & ~15u, nn = (n * n + 3u) & ~3u;
    L.s = 0;
    L.k = L.s + kF32Rows * D * 4u;
    L.q = L.k + n16 * D * 4u;
    L.v = L.q + n16 * D * 4u;
    L.p = L.v + n16 * kF32Rows * 4u;
    L.y = L.p + n * kF32Rows * 4u;
    L.u = L.y + n * kF32Rows * 4u;
    L.c = L.u + n * kF32Rows * 4u;
    L.w = L.c + nn * 4u;
    L.at = L.w + nn * 4u;
    L.sm = L.at + n * 64u;
    L.pk = L.sm + 5u * 256u;
    L.pu = L.pk + kF32Path * D * 4u;
    L.pg = L.pu + kF32Path * kF32Rows * 4u;
    L.bytes = L.pg + 256u;
    return L;
}

// One 16 x 16 tile D[i][j] = sum_k A[i][k] B[j][k] of two sets of 16 fp32 rows of 128 in LDS
// (chunk c of row r at c ^ (r % 16)) on the matrix cores.  Both operands are split into bf16
// hi + lo (split_hi_lo: |x - hi - lo| <= 2^-18 |x|) and each product is taken as
// hi.hi + hi.lo + lo.hi, dropping lo.lo (at most 2^-16 of it): three v_mfma_f32_16x16x32_bf16
// per 32-deep k-block, fp32 accumulation, one accumulator per kind of product (so the twelve
// products form three chains of four instead of one of twelve), every operand read first.
// Lane L gives row L % 16, k = 8 (L / 16) + 32 kb .. +7 of both operands (the same k order,
// so the sums are those of the plain product) and receives D[4 (L / 16) + e][L % 16],
// e = 0..3.
__device__ __forceinline__ f32x4_t f32_tile(const float* A, const float* Bm, int lane) {
    const int r = lane & 15;
    const int g = lane >> 4;
    f32x4_t a0[4], a1[4], b0[4], b1[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int c0 = (8 * kb + 2 * g) ^ r, c1 = (8 * kb + 2 * g + 1) ^ r;
        a0[kb] = *reinterpret_cast<const f32x4_t*>(A + r * D + 4 * c0);
        a1[kb] = *reinterpret_cast<const f32x4_t*>(A + r * D + 4 * c1);
        b0[kb] = *reinterpret_cast<const f32x4_t*>(Bm + r * D + 4 * c0);
        b1[kb] = *reinterpret_cast<const f32x4_t*>(Bm + r * D + 4 * c1);
    }
    f32x4_t acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        bf16x8_t ah, al, bh, bl;
        split_hi_lo(a0[kb], a1[kb], ah, al);
        split_hi_lo(b0[kb], b1[kb], bh, bl);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[2], 0, 0, 0);
    }
    return acc[0] + (acc[1] + acc[2]);
}

template <bool FUSED>
__global__ __launch_bounds__(kF32Threads)
void verify_f32_kernel(
    const float* __restrict__ S0, const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ parent, int H, int N, float* __restrict__ O,
    float* __restrict__ U, float* __restrict__ gamma, uint64_t* __restrict__ anc_out,
    int32_t* __restrict__ depth_out, int32_t* __restrict__ status, CommitInF32 cin)
{
    __shared__ uint64_t s_anc[MAXN];
    __shared__ float s_g[MAXN], s_rg[MAXN], s_beta[MAXN];
    __shared__ int s_dep[MAXN];
    __shared__ int s_path[MAXN];
    __shared__ int s_maxd, s_pdepth;
    extern __shared__ __align__(16) float dyn[];
    const F32Lds L = f32_lds(N);
    char* base = reinterpret_cast<char*>(dyn);
    const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dyn));
    float* Ss = reinterpret_cast<float*>(base + L.s);
    float* Ks = reinterpret_cast<float*>(base + L.k);
    float* Qs = reinterpret_cast<float*>(base + L.q);
    float* Vs = reinterpret_cast<float*>(base + L.v);
    float* Ps = reinterpret_cast<float*>(base + L.p);
    float* Ys = reinterpret_cast<float*>(base + L.y);
    float* Us = reinterpret_cast<float*>(base + L.u);
    float* Cs = reinterpret_cast<float*>(base + L.c);
    float* Ws = reinterpret_cast<float*>(base + L.w);
    uint8_t* At = reinterpret_cast<uint8_t*>(base + L.at);
    const int* SMi = reinterpret_cast<const int*>(base + L.sm);
    const float* SMf = reinterpret_cast<const float*>(base + L.sm);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x / kF32Blocks;
    const int blk = blockIdx.x - bh * kF32Blocks;
    const int r0 = blk * kF32Rows;
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;
    const size_t nstride = static_cast<size_t>(H) * D;   // floats between nodes of one head
    const float* Kh = K + (node0 * H + h) * D;
    const float* Qh = Q + (node0 * H + h) * D;
    const float* Vh = V + (node0 * H + h) * D + r0;
    const uint32_t un = static_cast<uint32_t>(N);
    const uint32_t ln = static_cast<uint32_t>(lane) < un ? static_cast<uint32_t>(lane) : 0u;

    // ---- every input in transfers issued at once.  Wave 0 gathers the parents, alphas and
    // betas (fused: wave 1 the previous tree and accepted node), waits for those alone and walks
    // its tree while the rows land; the rows are dealt round-robin to the other waves: 8
    // transfers of S rows (two rows each), ceil(N/2) of key rows and of query rows, ceil(N/16)
    // of value slices and (fused, previous tree of up to 16 nodes) ceil(Np/2) of K_prev rows,
    // one of U_prev slices and one gather of gammas.  Lanes past the last node load node 0
    // into slots nobody reads.
    const int nr2 = (N + 1) >> 1;
    const int nv = (N + 15) >> 4;
    const int npk = FUSED && cin.Np <= kF32Path ? (cin.Np + 1) >> 1 : 0;
    {
        constexpr int kFirstRowWave = FUSED ? 2 : 1;
        const int jobs = 8 + 2 * nr2 + nv + (npk > 0 ? npk + 2 : 0);
        const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
        const uint32_t c32 = static_cast<uint32_t>(lane) & 31u;
        if (wave == 0) {
            dma_x1(parent + node0, 4u * ln, lds + L.sm);
            dma_x1(alpha + node0 * H + h, 4u * ln * static_cast<uint32_t>(H), lds + L.sm + 256u);
            dma_x1(beta + node0 * H + h, 4u * ln * static_cast<uint32_t>(H), lds + L.sm + 512u);
        } else if (FUSED && wave == 1) {
            const uint32_t n = static_cast<uint32_t>(lane) < static_cast<uint32_t>(cin.Np)
                                   ? static_cast<uint32_t>(lane) : 0u;
            dma_x1(cin.parent + static_cast<size_t>(b) * cin.Np, 4u * n, lds + L.sm + 768u);
            dma_x1(cin.accepted + b, 0u, lds + L.sm + 1024u);
        } else {
            for (int j = wave - kFirstRowWave; j < jobs; j += kF32Waves - kFirstRowWave) {
                if (j < 8) {
                    const uint32_t r = 2u * j + hl;
                    dma_x4(S0 + static_cast<size_t>(bh) * D * D,
                           ((r0 + r) * D + 4u * (c32 ^ (r & 15u))) * 4u, lds + L.s + 1024u * j);
                } else if (j < 8 + 2 * nr2) {
                    const int jj = j - 8;
                    const bool is_q = jj >= nr2;
                    const uint32_t t = 2u * (is_q ? jj - nr2 : jj) + hl;
                    dma_x4(is_q ? Qh : Kh,
                           static_cast<uint32_t>((t < un ? t : 0u) * nstride * 4u) + 16u * (c32 ^ (t & 15u)),
                           lds + (is_q ? L.q : L.k) + 1024u * (is_q ? jj - nr2 : jj));
                } else if (j < 8 + 2 * nr2 + nv) {
                    const int jj = j - 8 - 2 * nr2;
                    const uint32_t t = 16u * jj + (static_cast<uint32_t>(lane) >> 2);
                    dma_x4(Vh, static_cast<uint32_t>((t < un ? t : 0u) * nstride * 4u) +
                                   16u * (static_cast<uint32_t>(lane) & 3u),
                           lds + L.v + 1024u * jj);
                } else {
                    // the previous tree's rows by node: K_prev rows (two per transfer), the
                    // block's U_prev slices (16 nodes per transfer), gammas (lane = node)
                    const size_t p0 = static_cast<size_t>(b) * cin.Np;
                    const uint32_t unp = static_cast<uint32_t>(cin.Np);
                    const int gp = j - 8 - 2 * nr2 - nv;
                    if (gp < npk) {
                        const uint32_t n = 2u * gp + hl;
                        dma_x4(cin.K + (p0 * H + h) * D,
                               static_cast<uint32_t>((n < unp ? n : 0u) * nstride * 4u) + 16u * c32,
                               lds + L.pk + 1024u * gp);
                    } else if (gp == npk) {
                        const uint32_t n = static_cast<uint32_t>(lane) >> 2;
                        dma_x4(cin.U + (p0 * H + h) * D + r0,
                               static_cast<uint32_t>((n < unp ? n : 0u) * nstride * 4u) +
                                   16u * (static_cast<uint32_t>(lane) & 3u),
                               lds + L.pu);
                    } else {
                        const uint32_t n = static_cast<uint32_t>(lane) < unp ? static_cast<uint32_t>(lane) : 0u;
                        dma_x1(cin.gamma + p0 * H + h, 4u * n * static_cast<uint32_t>(H), lds + L.pg);
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);              // this wave's own transfers
    }

    // ---- tree walk (wave 0, lane = node); with FUSED also the previous step's path (wave 1)
    if (wave == 0) {
        const int t = lane;
        int p = t < N ? SMi[t] : -1;
        const bool bad = t < N && (p < -1 || p >= t);
        if (bad) p = -1;
        uint64_t am = t < N ? (1ull << t) : 0ull;
        float g = t < N ? SMf[64 + t] : 1.0f;
        int j = p;
        for (int r = 0; (1 << r) < N; ++r) {       // ceil(log2 N) rounds: depth <= N
            const int src = j < 0 ? t : j;
            const uint64_t aj = shfl_u64(am, src);
            const float gj = __shfl(g, src);
            const int jj = __shfl(j, src);
            if (j >= 0) { am |= aj; g *= gj; j = jj; }
        }
        if (bad) report(status, TREEWY_ETREE);
        const int depth = __popcll(am);
        int dm = 0;                                  // the largest depth, bit by bit (ballots)
#pragma unroll
        for (int bit = 32; bit >= 1; bit >>= 1)
            if (__ballot(t < N && depth >= dm + bit)) dm += bit;
        if (t == 0) s_maxd = dm;
        if (t < N) {
            s_anc[t] = am;
            s_g[t] = g;
            s_rg[t] = 1.0f / g;
            s_beta[t] = SMf[128 + t];
            s_dep[t] = depth;
            uint64_t m = am;                         // ancestors-or-self, root first
            for (int i = 0; m != 0ull; ++i) {
                At[t * 64 + i] = static_cast<uint8_t>(__ffsll(static_cast<unsigned long long>(m)) - 1);
                m &= m - 1ull;
            }
            if (blk == 0) {
                gamma[(node0 + t) * H + h] = g;
                if (h == 0) {
                    if (anc_out) anc_out[node0 + t] = am;
                    if (depth_out) depth_out[node0 + t] = depth;
                }
            }
        }
    } else if (FUSED && wave == 1) {
        const int p_raw = lane < cin.Np ? SMi[192 + lane] : -1;
        const PathInfo pi = fused_path(p_raw, SMi[256], cin.Np, lane, blk == 0 && h == 0, status);
        if (lane == 0) s_pdepth = pi.depth;
        if (lane < pi.depth) s_path[lane] = pi.pn;
    }
    lds_barrier();                                   // every transfer landed; tree and path
                                                     // visible to all waves

    // ---- the previous step's commit on this block's rows (FUSED), written back to S; lane
    // (row tid / 16, columns 8 (tid % 16) .. +7); the path rows come 16 nodes per batch
    if constexpr (FUSED) {
        const int pd = s_pdepth;
        if (pd > 0) {
            const size_t p0 = static_cast<size_t>(b) * cin.Np;
            const int r = tid >> 4;
            const int k0 = 8 * (tid & 15);
            const float* PK = reinterpret_cast<const float*>(base + L.pk);
            const float* PU = reinterpret_cast<const float*>(base + L.pu);
            const float* PG = reinterpret_cast<const float*>(base + L.pg);
            // rows staged by node with the inputs (previous tree of up to 16 nodes), else
            // fetched here by path position
            const bool by_node = cin.Np <= kF32Path;
            float ga = 1.0f;
            // the lane's two 16-byte chunks of row r, where the swizzle put them
            const int p0c = (k0 >> 2) ^ r, p1c = ((k0 >> 2) + 1) ^ r;
            float4 s0 = *reinterpret_cast<const float4*>(Ss + r * D + 4 * p0c);
            float4 s1 = *reinterpret_cast<const float4*>(Ss + r * D + 4 * p1c);
            for (int q0 = 0; q0 < pd; q0 += kF32Path) {
                const int cnt = pd - q0 < kF32Path ? pd - q0 : kF32Path;
                const int nk = (cnt + 1) >> 1;
                const int jobs = by_node ? 0 : nk + 1 + (q0 == 0 ? 1 : 0);
                for (int j = wave; j < jobs; j += kF32Waves) {
                    if (j < nk) {
                        const int q = 2 * j + (lane >> 5);
                        const uint32_t n = static_cast<uint32_t>(s_path[q0 + (q < cnt ? q : 0)]);
                        dma_x4(cin.K + (p0 * H + h) * D,
                               static_cast<uint32_t>(n * nstride * 4u) + 16u * (static_cast<uint32_t>(lane) & 31u),
                               lds + L.pk + 1024u * j);
                    } else if (j == nk) {
                        const int q = lane >> 2;
                        const uint32_t n = static_cast<uint32_t>(s_path[q0 + (q < cnt ? q : 0)]);
                        dma_x4(cin.U + (p0 * H + h) * D + r0,
                               static_cast<uint32_t>(n * nstride * 4u) + 16u * (static_cast<uint32_t>(lane) & 3u),
                               lds + L.pu);
                    } else {
                        const int n = s_path[lane < pd ? lane : 0];
                        dma_gather_x1(cin.gamma + (p0 + n) * H + h, lds + L.pg);
                    }
                }
                if (!by_node) {
                    __builtin_amdgcn_s_waitcnt(0);
                    lds_barrier();
                }
                if (q0 == 0) {
                    ga = PG[by_node ? s_path[pd - 1] : pd - 1];
                    s0 = make_float4(ga * s0.x, ga * s0.y, ga * s0.z, ga * s0.w);
                    s1 = make_float4(ga * s1.x, ga * s1.y, ga * s1.z, ga * s1.w);
                }
#pragma unroll 4
                for (int q = 0; q < cnt; ++q) {
                    const int ig = by_node ? s_path[q0 + q] : q0 + q;   // gamma slot
                    const int ir = by_node ? s_path[q0 + q] : q;        // row slot
                    const float c = ga / PG[ig] * PU[ir * kF32Rows + r];
                    const float4 k_lo = *reinterpret_cast<const float4*>(PK + ir * D + k0);
                    const float4 k_hi = *reinterpret_cast<const float4*>(PK + ir * D + k0 + 4);
                    s0 = make_float4(s0.x + c * k_lo.x, s0.y + c * k_lo.y, s0.z + c * k_lo.z, s0.w + c * k_lo.w);
                    s1 = make_float4(s1.x + c * k_hi.x, s1.y + c * k_hi.y, s1.z + c * k_hi.z, s1.w + c * k_hi.w);
                }
                if (!by_node) lds_barrier();           // the batch is read: refill
            }
            *reinterpret_cast<float4*>(Ss + r * D + 4 * p0c) = s0;
            *reinterpret_cast<float4*>(Ss + r * D + 4 * p1c) = s1;
            float* dst = cin.S + (static_cast<size_t>(bh) * D + r0 + r) * D + k0;
            *reinterpret_cast<float4*>(dst) = s0;
            *reinterpret_cast<float4*>(dst + 4) = s1;
            lds_barrier();
        }
    }

    // ---- matrix-core tiles, dealt round-robin to the four waves: P^T and Y^T of this
    // block's rows (node tiles ct), and the Gram tiles K K^T (rt >= ct) and K Q^T (rt <= ct)
    {
        const int nt = (N + 15) >> 4;
        const int ntri = nt * (nt + 1) / 2;
        const int tiles = 2 * nt + 2 * ntri;
        const int col = lane & 15;
        const int rq = 4 * (lane >> 4);
        for (int tl = wave; tl < tiles; tl += kF32Waves) {
            int kind, rt = 0, ct;
            if (tl < 2 * nt) {
                kind = tl < nt ? 0 : 1;                  // 0: P, 1: Y
                ct = tl < nt ? tl : tl - nt;
            } else {
                const int g = tl - 2 * nt;
                kind = g < ntri ? 2 : 3;                 // 2: k.k (rt >= ct), 3: k.q (rt <= ct)
                int x = g < ntri ? g : g - ntri;
                while (x > rt) { x -= rt + 1; ++rt; }    // the x-th pair of row rt, 0 <= x <= rt
                ct = x;
                if (kind == 3) { const int y = rt; rt = ct; ct = y; }
            }
            const float* Am = kind <= 1 ? Ss : Ks + 16 * rt * D;
            const float* Bm = (kind == 1 || kind == 3 ? Qs : Ks) + 16 * ct * D;
            const f32x4_t d = f32_tile(Am, Bm, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = rq + e;                    // row of the tile
                const int jn = 16 * ct + col;            // node of its column
                if (kind <= 1) {
                    if (jn < N) (kind == 0 ? Ps : Ys)[jn * kF32Rows + i] = d[e];
                } else if (kind == 2) {
                    const int tn = 16 * rt + i;
                    if (tn < N && jn < N) Cs[tn * N + jn] = d[e];     // k_t . k_i
                } else {
                    const int an = 16 * rt + i;
                    if (an < N && jn < N) Ws[jn * N + an] = d[e];     // k_a . q_t
                }
            }
        }
    }
    lds_barrier();

    const int maxd = s_maxd;
    if (N * kF32Rows <= 64) {
        // a block's (node, row) pairs fit one wave: one pair per lane of wave 0, which takes the
        // right-hand sides, the levels of the substitution and the readout alone.  A wave's LDS
        // accesses take effect in issue order, so the levels need no workgroup barrier.
        if (wave != 0) return;
        const int x = lane;
        const bool ok = x < N * kF32Rows;
        const int t = ok ? x / kF32Rows : 0;
        const int r = x - t * kF32Rows;
        // the node's coefficients first (N <= 4: at most 4 ancestors-or-self), so that every
        // level of the substitution is one LDS round trip
        const int dep = ok ? s_dep[t] : 0;
        const float gt = s_g[t], bgt = s_beta[t] * gt;
        int anc[4];
        float cs[4], cw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = j < dep ? At[t * 64 + j] : t;
            anc[j] = i * kF32Rows + r;
            cs[j] = j < dep - 1 ? bgt * s_rg[i] * Cs[t * N + i] : 0.f;
            cw[j] = j < dep ? gt * s_rg[i] * Ws[t * N + i] : 0.f;
        }
        float u = ok ? s_beta[t] * (Vs[x] - gt * Ps[x]) : 0.f;
        if (ok) Us[x] = u;
        for (int d = 1; d < maxd; ++d) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // level d - 1 written
            if (ok && dep > d) {
                u -= cs[d - 1] * Us[anc[d - 1]];
                Us[x] = u;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (ok) {
            float o = gt * Ys[x];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < dep) o += cw[j] * Us[anc[j]];
            const size_t out = (node0 + t) * nstride + h * D + r0 + r;
            O[out] = o;
            U[out] = u;
        }
        return;
    }
    // ---- right-hand sides R[t][r] = b_t (v_t[r] - g_t P[t][r])
    for (int x = tid; x < N * kF32Rows; x += kF32Threads) {
        const int t = x / kF32Rows;
        Us[x] = s_beta[t] * (Vs[x] - s_g[t] * Ps[x]);
    }
    lds_barrier();
    // ---- forward substitution, level by level
    for (int d = 1; d < maxd; ++d) {
        for (int x = tid; x < N * kF32Rows; x += kF32Threads) {
            const int t = x / kF32Rows, r = x - t * kF32Rows;
            if (s_dep[t] > d) {
                const int a = At[t * 64 + d - 1];
                Us[x] -= s_beta[t] * s_g[t] * s_rg[a] * Cs[t * N + a] * Us[a * kF32Rows + r];
            }
        }
        lds_barrier();
    }
    // ---- readout O[t] = g_t Y[t] + sum over i ancestor-or-self of t of (g_t/g_i)(k_i.q_t) U[i]
    for (int x = tid; x < N * kF32Rows; x += kF32Threads) {
        const int t = x / kF32Rows, r = x - t * kF32Rows;
        float o = s_g[t] * Ys[x];
        for (int j = 0; j < s_dep[t]; ++j) {
            const int i = At[t * 64 + j];
            o += s_g[t] * s_rg[i] * Ws[t * N + i] * Us[i * kF32Rows + r];
        }
        const size_t out = (node0 + t) * nstride + h * D + r0 + r;
        O[out] = o;
        U[out] = Us[x];
    }
}

// ---------------------------------------------------------------------------------------
// fp32 inputs on trees of up to four nodes (and, fused, a previous tree of up to four): the
// same eight workgroups of 16 value rows per head, with everything after the transfers in
// registers.  Lane (r = tid / 16, c = tid % 16) owns columns 8c .. 8c + 7 of state row
// r0 + r.  Every lane derives the (tiny) trees from the staged parents itself: ancestor
// masks in topological order (parents precede children), gates as products.  It commits its
// eight state values (S_a = g_a S + sum over the path of (g_a / g_i) U_prev[i][r] k_i), takes
// its partial dot products with the keys and queries (P[t] = S_r . k_t, Y[t] = S_r . q_t over
// its eight columns) and sums them over the row's 16 lanes with DPP adds (quad permutes,
// half-row and row mirrors); the Gram entries k_t . k_i and k_i . q_t, the same for every
// row, are split over the wave's four rows and read back as wave-uniform values.  Each row's
// 16 lanes then hold the whole row of P and Y and the whole Gram matrix and solve the row's
// nodes in order (paper §3, Eq. 2 and the readout), in fp32 FMAs:
// U[t] = b_t (v_t - g_t P[t]) - sum over strict ancestors of b_t (g_t/g_i)(k_t.k_i) U[i],
// O[t] = g_t Y[t] + sum over ancestors-or-self of (g_t/g_i)(k_i.q_t) U[i]; lane c = t writes
// node t's O and U.  After the transfers the only LDS accesses are batches of operand reads,
// and no barrier follows: at one head the step is a chain of latencies, and this shortens it
// to the transfers and a few dependent register phases.

constexpr int kTinyN = 4;                       // nodes (and previous nodes) of this form

// v moved across lanes by the DPP control CTRL (all rows and banks, no bound control).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// The sum of v over the 16 lanes of a row (lanes 16q .. 16q + 15), in every one of them.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xb1>(v);                      // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp_mov<0x4e>(v);                      // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp_mov<0x141>(v);                     // row_half_mirror: the other quad of eight
    v += dpp_mov<0x140>(v);                     // row_mirror: the other half of sixteen
    return v;
}

template <bool FUSED>
__global__ __launch_bounds__(kF32Threads)
void verify_f32_tiny_kernel(
    const float* __restrict__ S0, const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ parent, int H, int N, float* __restrict__ O,
    float* __restrict__ U, float* __restrict__ gamma, uint64_t* __restrict__ anc_out,
    int32_t* __restrict__ depth_out, int32_t* __restrict__ status, CommitInF32 cin)
{
    // staged inputs (transfer destinations: whole 1 KB wave loads, 256 B gathers)
    __shared__ __align__(16) float Ss[kF32Rows * D];     // this block's 16 state rows
    __shared__ __align__(16) float Ks[kTinyN * D];       // key rows
    __shared__ __align__(16) float Qs[kTinyN * D];       // query rows
    __shared__ __align__(16) float PKs[kTinyN * D];      // previous keys (fused)
    __shared__ __align__(16) float Vs[256];              // value slices [node][16]
    __shared__ __align__(16) float PUs[256];             // previous U slices [node][16] (fused)
    __shared__ __align__(16) int32_t SMi[6 * 64];        // parent, alpha, beta, previous parent,
                                                         // accepted, previous gamma
    const float* SMf = reinterpret_cast<const float*>(SMi);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x / kF32Blocks;
    const int blk = blockIdx.x - bh * kF32Blocks;
    const int r0 = blk * kF32Rows;
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;
    const size_t nstride = static_cast<size_t>(H) * D;   // floats between nodes of one head
    const uint32_t un = static_cast<uint32_t>(N);
    const int Np = FUSED ? cin.Np : 0;
    const uint32_t unp = static_cast<uint32_t>(Np);
    const size_t p0 = static_cast<size_t>(b) * Np;

    // ---- every input in transfers issued at once, then each wave waits for its own
    {
        const uint32_t ln = static_cast<uint32_t>(lane) < un ? static_cast<uint32_t>(lane) : 0u;
        const uint32_t lnp = static_cast<uint32_t>(lane) < unp ? static_cast<uint32_t>(lane) : 0u;
        const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
        const uint32_t c32 = static_cast<uint32_t>(lane) & 31u;
        const uint32_t q4 = static_cast<uint32_t>(lane) >> 2;       // slices: node of the lane
        const uint32_t s4 = 16u * (static_cast<uint32_t>(lane) & 3u);
        const uint32_t lds_sm = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(SMi));
        const float* Kh = K + (node0 * H + h) * D;
        const float* Qh = Q + (node0 * H + h) * D;
        // 8 S rows transfers, 2 + 2 key/query, 1 value slices, 3 gathers; fused: 2 previous
        // key rows, 1 previous U slices, 3 gathers
        const int jobs = FUSED ? 22 : 16;
        for (int j = wave; j < jobs; j += kF32Waves) {
            if (j < 8) {
                const uint32_t rr = 2u * j + hl;
                dma_x4(S0 + static_cast<size_t>(bh) * D * D, ((r0 + rr) * D + 4u * c32) * 4u,
                       static_cast<uint32_t>(reinterpret_cast<uintptr_t>(Ss)) + 1024u * j);
            } else if (j < 12) {
                const bool is_q = j >= 10;
                const uint32_t t = 2u * (j - (is_q ? 10 : 8)) + hl;
                dma_x4(is_q ? Qh : Kh, static_cast<uint32_t>((t < un ? t : 0u) * nstride * 4u) + 16u * c32,
                       static_cast<uint32_t>(reinterpret_cast<uintptr_t>(is_q ? Qs : Ks)) +
                           1024u * (j - (is_q ? 10 : 8)));
            } else if (j == 12) {
                dma_x4(V + (node0 * H + h) * D + r0,
                       static_cast<uint32_t>((q4 < un ? q4 : 0u) * nstride * 4u) + s4,
                       static_cast<uint32_t>(reinterpret_cast<uintptr_t>(Vs)));
            } else if (j == 13) {
                dma_x1(parent + node0, 4u * ln, lds_sm);
            } else if (j == 14) {
                dma_x1(alpha + node0 * H + h, 4u * ln * static_cast<uint32_t>(H), lds_sm + 256u);
            } else if (j == 15) {
                dma_x1(beta + node0 * H + h, 4u * ln * static_cast<uint32_t>(H), lds_sm + 512u);
            } else if (j < 18) {
                const uint32_t n = 2u * (j - 16) + hl;
                dma_x4(cin.K + (p0 * H + h) * D,
                       static_cast<uint32_t>((n < unp ? n : 0u) * nstride * 4u) + 16u * c32,
                       static_cast<uint32_t>(reinterpret_cast<uintptr_t>(PKs)) + 1024u * (j - 16));
            } else if (j == 18) {
                dma_x4(cin.U + (p0 * H + h) * D + r0,
                       static_cast<uint32_t>((q4 < unp ? q4 : 0u) * nstride * 4u) + s4,
                       static_cast<uint32_t>(reinterpret_cast<uintptr_t>(PUs)));
            } else if (j == 19) {
                dma_x1(cin.parent + p0, 4u * lnp, lds_sm + 768u);
            } else if (j == 20) {
                dma_x1(cin.accepted + b, 0u, lds_sm + 1024u);
            } else {
                dma_x1(cin.gamma + p0 * H + h, 4u * lnp * static_cast<uint32_t>(H), lds_sm + 1280u);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
    }
    lds_barrier();

    const int r = tid >> 4;                     // row r0 + r
    const int c = tid & 15;                     // columns 8c .. 8c + 7
    const bool reporter = blk == 0 && tid == 0;

    // ---- the Gram entries first: they need the key and query rows only
    // the Gram entries (the same for every row): k_i . q_t (i <= t) and k_t . k_i (i < t),
    // 16 pairs; each row of the wave takes four (its lanes read those pairs' rows), and the
    // sums are read back from the four rows as wave-uniform values.  Pair pp is (i, t) =
    // (0,0) (0,1) (1,1) (0,2) (1,2) (2,2) (0,3) (1,3) (2,3) (3,3) for k_i . q_t, then (t, i) =
    // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2) for k_t . k_i: first index in nibble pp of kPairA,
    // second in nibble pp of kPairB.
    float G[16];
    {
        constexpr uint64_t kPairA = 0x3332213210210100ull;
        constexpr uint64_t kPairB = 0x2101003333222110ull;
        const int q = (tid >> 4) & 3;           // this lane's row within the wave
        float part[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pp = 4 * q + j;
            const int ia = static_cast<int>((kPairA >> (4 * pp)) & 15u);
            const int ib = static_cast<int>((kPairB >> (4 * pp)) & 15u);
            const float* ra = Ks + ia * D + 8 * c;
            const float* rb = (pp < 10 ? Qs : Ks) + ib * D + 8 * c;
            const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(ra);
            const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(ra + 4);
            const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(rb);
            const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(rb + 4);
            float x = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) x += a0[e] * b0[e] + a1[e] * b1[e];
            part[j] = row16_sum(x);
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                G[4 * qq + j] = __int_as_float(
                    __builtin_amdgcn_readlane(__float_as_int(part[j]), 16 * qq));
    }
    // ---- this step's tree, in every lane
    // (every staged slot holds a real node's words: slots past N repeat node 0, so all are
    // read at once and the ones past N are dropped)
    int par[kTinyN];
    float al[kTinyN], bt[kTinyN];
#pragma unroll
    for (int t = 0; t < kTinyN; ++t) {
        par[t] = SMi[t];
        al[t] = SMf[64 + t];
        bt[t] = t < N ? SMf[128 + t] : 0.0f;
    }
    uint32_t anc[kTinyN];
    float g[kTinyN];
    bool bad = false;
#pragma unroll
    for (int t = 0; t < kTinyN; ++t) {
        int p = par[t];
        if (t < N && (p < -1 || p >= t)) { bad = true; p = -1; }
        uint32_t ap = 0u;
        float gp = 1.0f;
#pragma unroll
        for (int i = 0; i < t; ++i)
            if (p == i) { ap = anc[i]; gp = g[i]; }
        anc[t] = t < N ? (ap | (1u << t)) : 0u;
        g[t] = t < N ? al[t] * gp : 1.0f;
    }
    if (bad && reporter) report(status, TREEWY_ETREE);
    if (blk == 0 && tid < N) {
        gamma[(node0 + tid) * H + h] = g[tid];
        if (h == 0) {
            uint64_t m = 0ull;
            int dd = 0;
#pragma unroll
            for (int t = 0; t < kTinyN; ++t)
                if (t == tid) { m = anc[t]; dd = __popc(anc[t]); }
            if (anc_out) anc_out[node0 + tid] = m;
            if (depth_out) depth_out[node0 + tid] = dd;
        }
    }

    // ---- this lane's eight state values, committed (fused)
    float sv[8];
    {
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(Ss + r * D + 8 * c);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(Ss + r * D + 8 * c + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { sv[e] = x0[e]; sv[4 + e] = x1[e]; }
    }
    if constexpr (FUSED) {
        // the previous tree's ancestor masks; a bad parent spoils every path through it
        // every operand first (slots past Np repeat node 0), the terms masked by the path
        int ppar[kTinyN];
        float pg[kTinyN], pu[kTinyN];
        f32x4_t pk0[kTinyN], pk1[kTinyN];
#pragma unroll
        for (int n = 0; n < kTinyN; ++n) {
            ppar[n] = SMi[192 + n];
            pg[n] = SMf[320 + n];
            pu[n] = PUs[n * kF32Rows + r];
            pk0[n] = *reinterpret_cast<const f32x4_t*>(PKs + n * D + 8 * c);
            pk1[n] = *reinterpret_cast<const f32x4_t*>(PKs + n * D + 8 * c + 4);
        }
        const int a = SMi[256];
        uint32_t panc[kTinyN], pbad = 0u;
#pragma unroll
        for (int n = 0; n < kTinyN; ++n) {
            int p = ppar[n];
            const bool bn = p < -1 || p >= n;
            if (bn) p = -1;
            uint32_t ap = 0u;
            bool bp = false;
#pragma unroll
            for (int i = 0; i < n; ++i)
                if (p == i) { ap = panc[i]; bp = (pbad >> i) & 1u; }
            panc[n] = n < Np ? (ap | (1u << n)) : 0u;
            if (n < Np && (bn || bp)) pbad |= 1u << n;
        }
        uint32_t path = 0u;
        if (a < -1 || a >= Np) {
            if (reporter) report(status, TREEWY_EACCEPT);
        } else if (a >= 0) {
            uint32_t m = 0u;
#pragma unroll
            for (int n = 0; n < kTinyN; ++n)
                if (n == a) m = panc[n];
            if ((pbad >> a) & 1u) {
                if (reporter) report(status, TREEWY_ETREE);
            } else {
                path = m;
            }
        }
        if (path != 0u) {
            float ga = 1.0f;
#pragma unroll
            for (int n = 0; n < kTinyN; ++n)
                if (n == a) ga = pg[n];
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[e] *= ga;
#pragma unroll
            for (int n = 0; n < kTinyN; ++n) {
                const float cu = ((path >> n) & 1u) ? ga * __builtin_amdgcn_rcpf(pg[n]) * pu[n] : 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sv[e] += cu * pk0[n][e];
                    sv[4 + e] += cu * pk1[n][e];
                }
            }
            float* dst = cin.S + (static_cast<size_t>(bh) * D + r0 + r) * D + 8 * c;
            *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{sv[0], sv[1], sv[2], sv[3]};
            *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{sv[4], sv[5], sv[6], sv[7]};
        }
    }

    // ---- partial dot products over the lane's eight columns, summed over the row
    float kv[kTinyN][8], qv[kTinyN][8];
#pragma unroll
    for (int t = 0; t < kTinyN; ++t) {
        const f32x4_t k0 = *reinterpret_cast<const f32x4_t*>(Ks + t * D + 8 * c);
        const f32x4_t k1 = *reinterpret_cast<const f32x4_t*>(Ks + t * D + 8 * c + 4);
        const f32x4_t q0 = *reinterpret_cast<const f32x4_t*>(Qs + t * D + 8 * c);
        const f32x4_t q1 = *reinterpret_cast<const f32x4_t*>(Qs + t * D + 8 * c + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kv[t][e] = k0[e];
            kv[t][4 + e] = k1[e];
            qv[t][e] = q0[e];
            qv[t][4 + e] = q1[e];
        }
    }
    float P[kTinyN], Y[kTinyN];
#pragma unroll
    for (int t = 0; t < kTinyN; ++t) {
        float p = 0.f, y = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p += sv[e] * kv[t][e];
            y += sv[e] * qv[t][e];
        }
        P[t] = row16_sum(p);
        Y[t] = row16_sum(y);
    }
    // KQ[i][t] = k_i . q_t, KK[t][i] = k_t . k_i from the pair list above
    auto KQv = [&](int i, int t) {
        return G[t * (t + 1) / 2 + i];
    };
    auto KKv = [&](int t, int i) {
        return G[10 + (t - 1) * t / 2 + i];
    };

    // ---- the row's solve and readout, in order (ancestors precede their descendants)
    float Uv[kTinyN], Ov[kTinyN];
#pragma unroll
    for (int t = 0; t < kTinyN; ++t) {
        Uv[t] = 0.f;
        Ov[t] = 0.f;
        if (t < N) {
            float u = bt[t] * (Vs[t * kF32Rows + r] - g[t] * P[t]);
#pragma unroll
            for (int i = 0; i < t; ++i)
                if ((anc[t] >> i) & 1u)
                    u -= bt[t] * g[t] * __builtin_amdgcn_rcpf(g[i]) * KKv(t, i) * Uv[i];
            Uv[t] = u;
            float o = g[t] * Y[t];
#pragma unroll
            for (int i = 0; i <= t; ++i)
                if ((anc[t] >> i) & 1u)
                    o += g[t] * __builtin_amdgcn_rcpf(g[i]) * KQv(i, t) * Uv[i];
            Ov[t] = o;
        }
    }
    if (c < N) {
        float uo = 0.f, oo = 0.f;
#pragma unroll
        for (int t = 0; t < kTinyN; ++t)
            if (t == c) { uo = Uv[t]; oo = Ov[t]; }
        const size_t out = (node0 + c) * nstride + h * D + r0 + r;
        O[out] = oo;
        U[out] = uo;
    }
}

// ---------------------------------------------------------------------------------------
// The small-tree verify kernel.  MODE 0 reads S0 as it is.  MODE 1 applies the previous
// step's commit to S on the way in and writes the committed rows back (see above).  MODE 2
// defers that write (a step of the log-structured commit, the deferred state writes the
// paper's Conclusion names as a next step): the committed state is kept as
// scale * (S + sum of logged rank-one terms).  Each item reads S, its log and the previous
// step's path; it forms the committed rows in LDS as in MODE 1 and verifies against them.
// When the log has room it appends the path's terms (divided by the new scale) instead of
// writing S. Otherwise (or when the path is longer than one LDS chunk) it writes the
// committed rows to S and empties the log.  Header words go to separate output buffers, so
// no item can see another item's update of the same sequence within one launch.

// The 16-byte chunk c of staged key row q (PK) sits at chunk c ^ head_pk_swizzle(q): the
// transposing reads of apply_terms take the same 32 bytes of 16 rows at once, which
// this spreads over the LDS banks (two rows per bank group instead of sixteen).
__device__ __forceinline__ uint32_t head_pk_swizzle(int q) {
    return 2u * (static_cast<uint32_t>(q) & 7u);
}

// Up to 16 rank-one terms applied to this wave's 16 rows of the state in LDS, on the matrix
// cores: S[r] <- c0 S[r] + sum over slots k < cnt of coef_k U_k[r] key_k^T, r = 16w + n (rows of
// the item in LDS, chunk c of row r at c ^ (r % 16)).  U_k is the slot's fp32 row of UStride
// values at byte u_area + 4 UStride k (r indexes it), key_k its bf16 row of 256 bytes at byte
// k_area + 256 k (k < k_rows staged; with Swizzled its 16-byte chunks sit at c ^
// head_pk_swizzle(k)).  Taken per 16-column tile jt as Delta^T = K^T (coef U) with
// v_mfma_f32_16x16x16_bf16: lane (g = lane / 16, n = lane % 16) gives A = key[4g + t][16 jt
// + n], t = 0..3 (one transposing LDS read of the key rows: the 16 lanes of a group address
// a block of 4 key rows x 16 columns and each receives one column), B = coef_{4g+t}
// U_{4g+t}[r] split into bf16 hi + lo (two products; the keys are exact in bf16,
// |x - hi - lo| <= 2^-18 |x|), C = c0 times the lane's 16-byte chunk 4 jt + g of row r, and
// D, the same four columns of row r after the update, goes back where C came from.  Slots
// past cnt are zero in both operands.  `coef` holds the lane's slots 4g..4g+3.
template <int UStride, bool Swizzled>
__device__ __forceinline__ void apply_terms(float* lds, uint32_t lds_addr, int cnt,
                                            const float (&coef)[4], float c0, uint32_t u_area,
                                            uint32_t k_area, int k_rows, int wave, int lane) {
    const int g = lane >> 4;
    const int n = lane & 15;
    const int r = 16 * wave + n;
    const float* PU = reinterpret_cast<const float*>(reinterpret_cast<const char*>(lds) + u_area);
    f32x4_t u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k = 4 * g + t;
        u[t] = k < cnt ? coef[t] * PU[k * UStride + r] : 0.f;
    }
    // the key row this lane addresses (clamped into the staged rows; masked below) and its
    // 8 bytes of each tile: chunk 2 jt + (n % 4) / 2 of the row, half n % 2
    const int qrow = 4 * g + (n >> 2) < k_rows ? 4 * g + (n >> 2) : 0;
    const uint32_t sw = Swizzled ? head_pk_swizzle(qrow) : 0u;
    const uint32_t arow = lds_addr + k_area + 256u * static_cast<uint32_t>(qrow) + 8u * static_cast<uint32_t>(n & 1);
    const uint32_t h2 = static_cast<uint32_t>(n & 3) >> 1;
    // every read first (the writes below may alias them as far as the compiler knows)
    i16x4_t a[D / 16];
    f32x4_t c[D / 16];
#pragma unroll
    for (int jt = 0; jt < D / 16; ++jt)
        a[jt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4_t*>(
            static_cast<uintptr_t>(arow + 16u * ((2u * jt + h2) ^ sw))));
#pragma unroll
    for (int jt = 0; jt < D / 16; ++jt)
        c[jt] = *reinterpret_cast<const f32x4_t*>(lds + r * D + 4 * ((4 * jt + g) ^ (r & 15)));
    const bf16x4_t uh = __builtin_convertvector(u, bf16x4_t);
    const u32x2_t hw = __builtin_bit_cast(u32x2_t, uh);
    const f32x4_t rem = {u[0] - __uint_as_float(hw[0] << 16), u[1] - __uint_as_float(hw[0] & 0xffff0000u),
                         u[2] - __uint_as_float(hw[1] << 16), u[3] - __uint_as_float(hw[1] & 0xffff0000u)};
    const i16x4_t bh = __builtin_bit_cast(i16x4_t, uh);
    const i16x4_t bl = __builtin_bit_cast(i16x4_t, __builtin_convertvector(rem, bf16x4_t));
    const uint32_t m0 = (4 * g < cnt ? 0x0000ffffu : 0u) | (4 * g + 1 < cnt ? 0xffff0000u : 0u);
    const uint32_t m1 = (4 * g + 2 < cnt ? 0x0000ffffu : 0u) | (4 * g + 3 < cnt ? 0xffff0000u : 0u);
#pragma unroll
    for (int jt = 0; jt < D / 16; ++jt) {
        u32x2_t aw = __builtin_bit_cast(u32x2_t, a[jt]);
        aw[0] &= m0;
        aw[1] &= m1;
        const i16x4_t am = __builtin_bit_cast(i16x4_t, aw);
        c[jt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(am, bh, c0 * c[jt], 0, 0, 0);
        c[jt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(am, bl, c[jt], 0, 0, 0);
    }
#pragma unroll
    for (int jt = 0; jt < D / 16; ++jt)
        *reinterpret_cast<f32x4_t*>(lds + r * D + 4 * ((4 * jt + g) ^ (r & 15))) = c[jt];
}


// NFIX > 0: a form compiled for trees of exactly NFIX nodes (every mode on up to 8 nodes),
// whose LDS offsets, loop bounds and pointer-jumping rounds are constants; 0: N at run time.
template <int NCT, int MODE, int NFIX = 0>
__global__ __launch_bounds__(kSmallThreads)
__attribute__((amdgpu_waves_per_eu(kSmallWavesPerSimd<NCT, MODE>)))
void verify_small_kernel(
    const float* S0, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const float* __restrict__ alpha,
    const float* __restrict__ beta, const int32_t* __restrict__ parent, int H, int N_rt, int BH,
    float* __restrict__ O, float* __restrict__ U, float* __restrict__ gamma,
    uint64_t* __restrict__ anc_out, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ status, CommitIn cin, DeferLog dlog)
{
    const int N = NFIX > 0 ? NFIX : N_rt;
    constexpr bool FUSED = MODE != 0;
    constexpr bool DEFER = MODE == 2;
    constexpr bool TWO = small_two_sets(NCT, MODE); // two input sets, early refills
    // the deferred commit's terms on the matrix cores (apply_terms) on 9-16 nodes; on up
    // to 8 the vector-ALU form (the product's registers would spill at this kernel's budget
    // of three waves per SIMD)
    constexpr bool kMatrixDefer = DEFER && NCT == 2;
    constexpr int kGP = 16 * NCT;                   // G row pitch
    extern __shared__ __align__(16) float lds[];
    const SmallLds L = small_lds(N, NCT, MODE, DEFER ? dlog.Lmax : 0);
    const char* ldsb = reinterpret_cast<const char*>(lds);
    float* G = lds + L.g / 4;                       // G[m][n] = k_m . (k|q)_n
    const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keep it scalar
    const int col = lane & 15;                      // output column within a tile
    const int grp = lane >> 4;                      // 16-lane group: rows 4 grp .. 4 grp + 3
    const int base = lane & 48;                     // first lane of this 16-lane group
    const int t = col;                              // this lane's node in the tail
    const bool node_ok = t < N;
    const int nq4 = (N + 3) >> 2;
    const int grid = gridDim.x;
    const int slot = blockIdx.x;

    int bh, part;
    small_item(0, slot, grid, bh, part);
    if (bh >= BH) return;

    PathInfo cur{0ull, 0, 0};                       // this item's commit (FUSED)
    int cur_len = 0;                                // this item's log length (DEFER)
    if constexpr (FUSED) {
        // item 0's previous tree and accepted node (and log length) go out first, then its S
        // rows; the path is derived while the rows stream in, then its own rows (and log) and
        // item 0's other inputs (with item 1's accepted node and tree) follow
        int bh1, part1;
        small_item(1, slot, grid, bh1, part1);
        if (wave == 0) {
            fused_issue_index(cin, bh / H, lane, lds_addr + L.idx);
            dma_gather_x1(cin.accepted + bh / H, lds_addr + L.sm);
            if constexpr (DEFER) dma_x1(dlog.len_in + bh / H, 0u, lds_addr + L.il);
        }
        small_issue_s0<FUSED>(S0, lds, bh, part, wave, lane);
        __builtin_amdgcn_s_waitcnt(kWaitAllButEight);   // the gathers (the eight row loads go on)
        lds_barrier();
        cur = fused_path(lane < cin.Np ? reinterpret_cast<const int*>(ldsb + L.idx)[lane] : -1,
                         reinterpret_cast<const int*>(ldsb + L.sm)[48], cin.Np, lane,
                         wave == 0 && bh % H == 0 && part == 0, status);
        if constexpr (DEFER) {
            const int raw = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(ldsb + L.il)[0]);
            cur_len = log_len(raw, dlog.Lmax);
            if (raw != cur_len && wave == 0 && lane == 0 && bh % H == 0 && part == 0)
                report(status, TREEWY_ELOG);
        }
        lds_barrier();                              // index read by every wave: refill
        if (cur.depth > 0) fused_issue_path(cin, cur, 0, bh, part, H, wave, lane, lds_addr, L);
        if constexpr (DEFER) defer_issue_log(dlog, cur_len, bh, part, wave, lane, lds_addr, L);
        small_issue_inputs(Q, K, V, alpha, beta, parent, H, N, bh, part, wave, lane, lds_addr, L,
                           bh1 < BH ? cin.accepted + bh1 / H : nullptr);
        if (bh1 < BH && wave == 3) {
            fused_issue_index(cin, bh1 / H, lane, lds_addr + L.idx);
            if constexpr (DEFER) dma_x1(dlog.len_in + bh1 / H, 0u, lds_addr + L.il);
        }
    } else {
        small_issue_s0<FUSED>(S0, lds, bh, part, wave, lane);
        small_issue_inputs(Q, K, V, alpha, beta, parent, H, N, bh, part, wave, lane, lds_addr, L,
                           nullptr);
    }
    __builtin_amdgcn_s_waitcnt(0);                  // the first item: nothing else in flight

    uint32_t sb = 0;                                // this item's input set (TWO: 0 or L.set)
    for (int round = 0;; ) {
        const int b = bh / H;
        const int h = bh - b * H;
        const size_t node0 = static_cast<size_t>(b) * N;
        const int v0 = part * kSmallRows + 16 * wave + 4 * grp;   // this lane's value rows

        // This item's transfers have landed once at most the two stores of the previous item
        // (O and U, issued last) are still in flight: vector memory operations retire in issue
        // order, so vmcnt <= 2 covers everything else.
        __builtin_amdgcn_s_waitcnt(kWaitAllButTwoStores);
        lds_barrier();                              // ... for every wave; last item fully done

        int bh_n, part_n;
        small_item(round + 1, slot, grid, bh_n, part_n);
        const bool more = bh_n < BH;

        PathInfo nxt{0ull, 0, 0};
        int nxt_len = 0;
        if constexpr (TWO) {
            // the next item's path (its previous tree and accepted node came with this item's
            // transfers), then its inputs and path rows into the other set, with the previous
            // tree and accepted node of the item after it
            if (more) {
                const uint32_t sbn = sb ? 0u : L.set;
                nxt = fused_path(lane < cin.Np ? reinterpret_cast<const int*>(ldsb + sb + L.idx)[lane] : -1,
                                 reinterpret_cast<const int*>(ldsb + sb + L.sm)[48], cin.Np, lane,
                                 wave == 0 && bh_n % H == 0 && part_n == 0, status);
                int bh_2, part_2;
                small_item(round + 2, slot, grid, bh_2, part_2);
                small_issue_inputs(Q, K, V, alpha, beta, parent, H, N, bh_n, part_n, wave, lane,
                                   lds_addr + sbn, L, bh_2 < BH ? cin.accepted + bh_2 / H : nullptr);
                if (nxt.depth > 0)
                    fused_issue_path(cin, nxt, 0, bh_n, part_n, H, wave, lane, lds_addr + sbn, L);
                if (bh_2 < BH && wave == 3) fused_issue_index(cin, bh_2 / H, lane, lds_addr + sbn + L.idx);
            }
        }

        if constexpr (FUSED) {
            int len = 0;
            float gin = 1.0f;
            if constexpr (DEFER) {
                len = cur_len;
                gin = reinterpret_cast<const float*>(ldsb + sb + L.lg)[0];
            }
            const bool any = cur.depth > 0 || len > 0;
            // MODE 1 always writes S; MODE 2 only when the log cannot take the path's terms
            bool flush = true;
            if constexpr (DEFER) flush = len + cur.depth > dlog.Lmax || cur.depth > L.path;
            const float* PG = reinterpret_cast<const float*>(ldsb + sb + L.pg);
            const float ga = cur.depth > 0 ? PG[cur.depth - 1] : 1.0f;
            const float gs = gin * ga;              // the scale of S (and of the logged terms)
            if (any) {
                // S_a = gs (S + sum_j u~_j k_j^T) + sum over the path of (g_a / g_i) U_prev[i]
                // k_i^T (MODE 1: no log, gs = g_a), applied to this wave's 16 rows where they
                // sit in LDS, in the layout they arrived in (lane l: row 16w + 2i + l / 32,
                // 16-byte chunk l % 32, for i = 0..7), and written back to HBM from there when
                // flushing: every store is two whole 512-byte rows (the deferred form on 9-16
                // nodes applies the terms with apply_terms instead).  The path's gammas
                // are in LDS in path order (a is last).
                const float* PU = reinterpret_cast<const float*>(ldsb + sb + L.pu);
                const char* PK = ldsb + sb + L.pk;
                const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
                const uint32_t ch = static_cast<uint32_t>(lane) & 31u;   // values 4 ch .. 4 ch + 3
                const int nchunk = cur.depth > 0 ? (cur.depth + L.path - 1) / L.path : 1;
                if constexpr (kMatrixDefer) {
                    // the log's terms (one product: at most 16), then the path's, per chunk,
                    // on the matrix cores; the first product also scales S by gs
                    const int g = lane >> 4;
                    bool scaled = false;
                    if (len > 0) {
                        const float coef[4] = {gs, gs, gs, gs};
                        apply_terms<kSmallRows, false>(lds, lds_addr, len, coef, gs, sb + L.lu, sb + L.lk,
                                          4 * ((dlog.Lmax + 3) / 4), wave, lane);
                        scaled = true;
                    }
                    for (int ci = 0; ci < (cur.depth > 0 ? nchunk : 0); ++ci) {
                        const int q0 = ci * L.path;
                        if (ci > 0) {
                            // a path longer than one chunk: the next chunk, with a blocking wait
                            lds_barrier();
                            fused_issue_path(cin, cur, ci, bh, part, H, wave, lane, lds_addr + sb, L);
                            __builtin_amdgcn_s_waitcnt(0);
                            lds_barrier();
                        }
                        const int rem = cur.depth - q0;
                        const int cnt = rem < L.path ? rem : L.path;
                        float coef[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const int q = q0 + 4 * g + t;
                            coef[t] = ga * __builtin_amdgcn_rcpf(PG[q < 64 ? q : 0]);
                        }
                        apply_terms<kSmallRows, false>(lds, lds_addr, cnt, coef, scaled ? 1.0f : gs,
                                          sb + L.pu, sb + L.pk, L.path, wave, lane);
                        scaled = true;
                    }
                    if (flush) {
                        // the committed rows back to HBM as whole rows (this wave's own rows,
                        // written by its products above)
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const uint32_t r = 16u * wave + 2u * i + hl;
                            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(lds + r * D + 4 * (ch ^ (r & 15u)));
                            __builtin_nontemporal_store(
                                x, reinterpret_cast<f32x4_t*>(
                                       cin.S + (static_cast<size_t>(bh) * D + part * kSmallRows + r) * D + 4 * ch));
                        }
                    }
                }
                for (int ci = 0; ci < (kMatrixDefer ? 0 : nchunk); ++ci) {
                    const int q0 = ci * L.path;
                    if (ci > 0) {
                        // a path longer than one chunk: the next chunk, with a blocking wait
                        lds_barrier();
                        fused_issue_path(cin, cur, ci, bh, part, H, wave, lane, lds_addr + sb, L);
                        __builtin_amdgcn_s_waitcnt(0);
                        lds_barrier();
                    }
                    const int rem = cur.depth - q0;
                    const int cnt = rem < L.path ? rem : L.path;
                    f32x4_t x[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t r = 16u * wave + 2u * i + hl;
                        x[i] = *reinterpret_cast<const f32x4_t*>(lds + r * D + 4 * (ch ^ (r & 15u)));
                        if (ci == 0) x[i] *= gs;
                    }
                    if constexpr (DEFER) {
                        if (ci == 0) {
                            const float* LU = reinterpret_cast<const float*>(ldsb + sb + L.lu);
                            const char* LK = ldsb + sb + L.lk;
                            for (int q = 0; q < len; ++q) {
                                const uint2 kw = *reinterpret_cast<const uint2*>(LK + q * 256 + 8 * ch);
                                const f32x4_t kv = {__uint_as_float(kw.x << 16), __uint_as_float(kw.x & 0xffff0000u),
                                                    __uint_as_float(kw.y << 16), __uint_as_float(kw.y & 0xffff0000u)};
#pragma unroll
                                for (int i = 0; i < 8; ++i) {
                                    const float cu = gs * LU[q * kSmallRows + 16 * wave + 2 * i + hl];
                                    x[i] += cu * kv;
                                }
                            }
                        }
                    }
                    // the path's terms; with the fused commit the loop is unrolled over the
                    // chunk's slots, so that the reads of all its rows are issued together
                    auto path_term = [&](int q) {
                        const float cq = ga / PG[q0 + q];
                        const uint2 kw = *reinterpret_cast<const uint2*>(PK + q * 256 + 8 * ch);
                        const f32x4_t kv = {__uint_as_float(kw.x << 16), __uint_as_float(kw.x & 0xffff0000u),
                                            __uint_as_float(kw.y << 16), __uint_as_float(kw.y & 0xffff0000u)};
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const float cu = cq * PU[q * kSmallRows + 16 * wave + 2 * i + hl];
                            x[i] += cu * kv;
                        }
                    };
                    if constexpr (MODE == 1) {
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            if (q >= cnt) break;
                            path_term(q);
                        }
                    } else {
                        for (int q = 0; q < cnt; ++q) path_term(q);
                    }
                    const bool last = ci + 1 == nchunk;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t r = 16u * wave + 2u * i + hl;
                        *reinterpret_cast<f32x4_t*>(lds + r * D + 4 * (ch ^ (r & 15u))) = x[i];
                        if (last && flush)
                            __builtin_nontemporal_store(
                                x[i], reinterpret_cast<f32x4_t*>(
                                          cin.S + (static_cast<size_t>(bh) * D + part * kSmallRows + r) * D +
                                          4 * ch));
                    }
                }
                if constexpr (DEFER) {
                    if (!flush && cur.depth > 0 && wave == 0) {
                        // the path's terms join the log at rows len ..: this half of each
                        // u~ = (g_a / g_i) U_prev[i] / gs, and this half of each key row
                        const size_t row0 = static_cast<size_t>(bh) * dlog.Lmax + len;
                        for (int q = lane >> 4; q < cur.depth; q += 4) {
                            const int c4 = lane & 15;
                            const float cq = (ga / PG[q]) / gs;
                            const f32x4_t u = *reinterpret_cast<const f32x4_t*>(PU + q * kSmallRows + 4 * c4);
                            *reinterpret_cast<f32x4_t*>(dlog.U + (row0 + q) * D + part * kSmallRows + 4 * c4) = cq * u;
                        }
                        for (int q = lane >> 3; q < cur.depth; q += 8) {
                            const int c8 = lane & 7;
                            const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(PK + q * 256 + 128 * part + 16 * c8);
                            *reinterpret_cast<u32x4_t*>(dlog.K + (row0 + q) * D + part * kSmallRows + 8 * c8) = kv;
                        }
                    }
                }
            }
            if constexpr (DEFER) {
                // the header after this step: an emptied log has scale 1 and length 0
                if (wave == 0 && lane == 0 && part == 0) {
                    const bool emptied = any && flush;
                    dlog.scale_out[bh] = emptied ? 1.0f : gs;
                    if (h == 0) dlog.len_out[b] = emptied ? 0 : len + cur.depth;
                }
            }
        }

        // ---- MFMA operands of this wave's 16 rows (committed, with FUSED), split into bf16
        //      hi and lo: lane L takes row 16w + L % 16, values 32 ks + 8 (L / 16) .. +7.
        //      With two input sets the rows are taken here, and half of the wave's rows of
        //      the next item are requested at once (the other half before the walk).
        bf16x8_t ahi[4], alo[4];
        auto take_rows = [&]() {
            const int r = 16 * wave + col;
            const float* rowp = lds + r * D;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int c0 = 2 * grp + 8 * ks;
                split_hi_lo(*reinterpret_cast<const f32x4_t*>(rowp + 4 * (c0 ^ (r & 15))),
                            *reinterpret_cast<const f32x4_t*>(rowp + 4 * ((c0 + 1) ^ (r & 15))),
                            ahi[ks], alo[ks]);
            }
        };
        if constexpr (TWO) {
            take_rows();
            if (more) {
                __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);   // this wave's reads of its rows
                issue_s_pairs<FUSED>(S0, lds_addr, bh_n, part_n, 0, 2, wave, lane);   // half the rows
            }
        }

        // ---- this item's operands out of LDS
        const int my_par = node_ok ? reinterpret_cast<const int*>(ldsb + sb + L.sm)[t] : -1;
        const float my_alpha = node_ok ? reinterpret_cast<const float*>(ldsb + sb + L.sm)[16 + t] : 1.0f;
        const float my_beta = node_ok ? reinterpret_cast<const float*>(ldsb + sb + L.sm)[32 + t] : 0.0f;
        uint2 vraw = make_uint2(0u, 0u);
        if (node_ok) vraw = *reinterpret_cast<const uint2*>(ldsb + sb + L.v + t * 128 + 32 * wave + 8 * grp);
        bf16x8_t bfr[NCT][4];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            const int n = 16 * c + col;
            const int r = n < N ? n : (n < 2 * N ? 4 * nq4 + n - N : -1);
            const char* rowp = ldsb + sb + L.kq + 256 * (r < 0 ? 0 : r);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                u32x4_t w = {0u, 0u, 0u, 0u};
                if (r >= 0) w = *reinterpret_cast<const u32x4_t*>(rowp + 16 * ((4 * ks + grp) ^ (r & 15)));
                bfr[c][ks] = __builtin_bit_cast(bf16x8_t, w);
            }
        }
        if constexpr (FUSED && !TWO) {
            if (more) {
                nxt = fused_path(lane < cin.Np ? reinterpret_cast<const int*>(ldsb + L.idx)[lane] : -1,
                                 reinterpret_cast<const int*>(ldsb + L.sm)[48], cin.Np, lane,
                                 wave == 0 && bh_n % H == 0 && part_n == 0, status);
                if constexpr (DEFER) {
                    const int raw = __builtin_amdgcn_readfirstlane(
                        reinterpret_cast<const int*>(ldsb + L.il)[0]);
                    nxt_len = log_len(raw, dlog.Lmax);
                    if (raw != nxt_len && wave == 0 && lane == 0 && bh_n % H == 0 && part_n == 0)
                        report(status, TREEWY_ELOG);
                }
            }
        }

        // ---- tree walk, in every 16-lane group (lane = node t): pointer jumping as in
        //      tree_walk, ceil(log2 N) rounds (at most four for a small tree)
        uint32_t anc;
        float g_t, rg_t;
        {
            int p = my_par;
            const bool bad = node_ok && (p < -1 || p >= t);
            if (bad) p = -1;
            uint32_t am = node_ok ? (1u << t) : 0u;
            float g = node_ok ? my_alpha : 1.0f;
            int j = p;
            for (int r = 0; (1 << r) < N; ++r) {    // ceil(log2 N) rounds: depth <= N
                const int src = base | (j < 0 ? t : j);
                const uint32_t aj = __shfl(am, src);
                const float gj = __shfl(g, src);
                const int jj = __shfl(j, src);
                if (j >= 0) { am |= aj; g *= gj; j = jj; }
            }
            anc = am;
            g_t = g;
            rg_t = 1.0f / g;
            if (wave == 0 && grp == 0 && node_ok && part == 0) {
                if (bad) report(status, TREEWY_ETREE);
                gamma[(node0 + t) * H + h] = g;
                if (h == 0) {
                    if (anc_out) anc_out[node0 + t] = am;
                    if (depth_out) depth_out[node0 + t] = __popc(am);
                }
            }
        }

        // ---- wave 0: Gram matrix G = K [K;Q]^T (keys of tile 0 are the A operand) -> LDS
        if (wave == 0) {
            f32x4_t gacc[NCT];
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                gacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    bf16x8_t ka = bfr[0][ks];
                    if (col >= N) ka = bf16x8_t{};
                    gacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bfr[c][ks], gacc[c], 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) G[(4 * grp + e) * kGP + 16 * c + col] = gacc[c][e];
            }
        }

        if constexpr (!TWO) take_rows();
        lds_barrier();                              // operands read and G visible: refill
        ++round;
        if (more && !TWO) {
            issue_s_pairs<FUSED>(S0, lds_addr, bh_n, part_n, 0, 2, wave, lane);   // half the rows
            if constexpr (FUSED) {
                // item i + 1's inputs and path rows; item i + 2's accepted node and tree
                int bh_2, part_2;
                small_item(round + 1, slot, grid, bh_2, part_2);
                small_issue_inputs(Q, K, V, alpha, beta, parent, H, N, bh_n, part_n, wave, lane,
                                   lds_addr, L, bh_2 < BH ? cin.accepted + bh_2 / H : nullptr);
                if (nxt.depth > 0)
                    fused_issue_path(cin, nxt, 0, bh_n, part_n, H, wave, lane, lds_addr, L);
                if constexpr (DEFER)
                    defer_issue_log(dlog, nxt_len, bh_n, part_n, wave, lane, lds_addr, L);
                if (bh_2 < BH && wave == 3) {
                    fused_issue_index(cin, bh_2 / H, lane, lds_addr + L.idx);
                    if constexpr (DEFER) dma_x1(dlog.len_in + bh_2 / H, 0u, lds_addr + L.il);
                }
            } else {
                small_issue_inputs(Q, K, V, alpha, beta, parent, H, N, bh_n, part_n, wave, lane,
                                   lds_addr, L, nullptr);
            }
        }

        // ---- contractions on the matrix cores
        f32x4_t acc[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[ks], bfr[c][ks], acc[c], 0, 0, 0);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[ks], bfr[c][ks], acc[c], 0, 0, 0);
            }
        }

        // ---- per lane: node t, rows v0..v0+3
        float Yv[4];
        {
            // query t sits in column N + t: tile (N + t) / 16, lane (N + t) % 16.  Each source
            // lane s serves exactly one node (t = s - N in tile 0, or t = s + 16 - N in tile
            // 1), so it publishes that tile's value and one permute per row suffices.
            const int src = base | ((N + t) & 15);
            const int tile = (NCT > 1 && col < N) ? 1 : 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pub = NCT > 1 ? (tile ? acc[NCT > 1 ? 1 : 0][e] : acc[0][e]) : acc[0][e];
                Yv[e] = __shfl(pub, src);
            }
        }
        const float b_t = node_ok ? my_beta : 0.f;
        const float gg_t = node_ok ? g_t : 0.f;
        const float bg_t = b_t * gg_t;
        const float vv[4] = {__uint_as_float(vraw.x << 16), __uint_as_float(vraw.x & 0xffff0000u),
                             __uint_as_float(vraw.y << 16), __uint_as_float(vraw.y & 0xffff0000u)};
        float Uv[4], Ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Uv[e] = b_t * vv[e] - bg_t * acc[0][e];  // R[t] = b_t (v_t - g_t S0 k_t)
            Ov[e] = gg_t * Yv[e];                    // g_t S0 q_t
        }

        if (more)                                   // the other half of the next item's rows
            issue_s_pairs<FUSED>(S0, lds_addr, bh_n, part_n, 4, 2, wave, lane);

        // One walk down the ancestors serves both the forward substitution and the readout:
        // at step d the depth-d ancestor a of t is final (its own terms ended at step d - 1),
        // so its U enters both U[t] -= b_t (g_t/g_a)(k_t.k_a) U[a] and
        // O[t] += (g_t/g_a)(k_a.q_t) U[a].  The wave goes on while any lane has ancestors left.
        uint32_t m = anc & ~(1u << t);
        while (__any(m != 0u)) {
            const bool has = m != 0u;
            const int a = has ? __builtin_ctz(m) : t;
            m &= m - 1u;
            const float rg_a = __shfl(rg_t, base | a);
            // lanes without an ancestor left read entry 0 (their coefficient is zero)
            const float cs = has ? bg_t * rg_a * G[has ? t * kGP + a : 0] : 0.f;
            const float cw = has ? gg_t * rg_a * G[has ? a * kGP + N + t : 0] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = __shfl(Uv[e], base | a);
                Uv[e] -= cs * x;
                Ov[e] += cw * x;
            }
        }
        {
            const float cw = node_ok ? G[node_ok ? t * kGP + N + t : 0] : 0.f;   // g_t/g_t = 1
#pragma unroll
            for (int e = 0; e < 4; ++e) Ov[e] += cw * Uv[e];
        }
        // O and U rows of this head through buffer descriptors that span exactly its rows:
        // lanes without a node get an offset past the end, which the hardware drops.  The
        // stores are thus unconditional, so the compiler's wait at the next item's top can
        // leave them in flight.
        {
            const uint32_t span = static_cast<uint32_t>(((N - 1) * H + 1) * D * sizeof(float));
            const size_t row0 = (node0 * H + h) * D;
            const uint32_t off = node_ok ? static_cast<uint32_t>((t * H * D + v0) * sizeof(float)) : span;
            const f32x4_t ov = {Ov[0], Ov[1], Ov[2], Ov[3]};
            const f32x4_t uv = {Uv[0], Uv[1], Uv[2], Uv[3]};
            __builtin_amdgcn_raw_buffer_store_b128(
                ov, __builtin_amdgcn_make_buffer_rsrc(O + row0, 0, span, kRawBufferFlags), off, 0, (FUSED && !TWO) ? kStreamAux : 0);
            __builtin_amdgcn_raw_buffer_store_b128(
                uv, __builtin_amdgcn_make_buffer_rsrc(U + row0, 0, span, kRawBufferFlags), off, 0, (FUSED && !TWO) ? kStreamAux : 0);
        }
        if (!more) break;
        bh = bh_n;
        part = part_n;
        if constexpr (FUSED) {
            cur = nxt;
            cur_len = nxt_len;
        }
        if constexpr (TWO) sb = sb ? 0u : L.set;
    }
}

// ---------------------------------------------------------------------------------------
// Trees of 17 to 32 nodes, the plain verify: the persistent streaming design of the
// small-tree kernel, with NKT = 2 node tiles per lane (the fused and deferred steps on 17-64
// nodes, and the plain verify on 33-64, take the one-head-per-item kernel below).
//
// Output columns: keys at 0..N-1 (tiles 0..NKT-1), queries at 16 NKT + t (tiles NKT..2NKT-1),
// so lane L holds P[t] and Y[t] for the nodes t = 16 kt + L % 16 of every node tile kt, rows
// 16w + 4 (L / 16) .. +3.  Each wave walks the tree with lane = node (pointer jumping)
// and hands every lane its nodes' masks and gates by lane permutes.  The forward substitution
// and readout are the same ancestor walk as above; U of the ancestors is exchanged through a
// per-wave LDS scratch [32 nodes][16 rows] instead of lane permutes, because an ancestor may sit
// in another node tile.  A wave's LDS operations complete in issue order, so a value written
// at the end of step d - 1 is what other lanes of the wave read at step d.  The Gram matrix
// G = K [K;Q]^T (same column layout) is formed by waves 0..NKT-1 and staged in LDS.
//
// The item's key and query rows are sent into the S-row area once the rows have been taken
// into registers, and the contractions read them there; values, gates and tree are
// prefetched into registers.  The next item's S0 rows are requested once every wave is past
// the contractions.  Three workgroups per CU.

template <int NKT>
struct LargeLayout {
    static constexpr int kCols = 32 * NKT;                // G row pitch (keys | queries)
    static constexpr int kS0 = kSmallRows * D;            // floats
    static constexpr int kG = 16 * NKT * kCols;           // G [16 NKT][kCols]
    static constexpr int kU = 4 * 16 * NKT * 16;          // per wave [16 NKT nodes][16 rows]
    static constexpr int kTotal = kS0 + kG + kU;
    // s_waitcnt operand: vmcnt <= 2 NKT (the previous item's O and U stores), no other wait
    static constexpr int kWait = (2 * NKT) | (7 << 4) | (15 << 8);
};

// The item's key and query rows alone -> LDS at `lds` (the staged layout: keys in rows
// 0 .. 4 ceil(N/4) - 1, queries right after, 256 B rows, chunk c of row r at c ^ (r % 16)),
// 2 ceil(N/4) transfers of four rows dealt to the four waves.  At most 16 KiB (N <= 32).
__device__ __forceinline__ void large_issue_kq(const uint16_t* Q, const uint16_t* K, int H, int N,
                                               int bh, int wave, int lane, uint32_t lds) {
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;
    const uint32_t row_bytes = static_cast<uint32_t>(H) * D * 2;
    const uint16_t* Kh = K + (node0 * H + h) * D;
    const uint16_t* Qh = Q + (node0 * H + h) * D;
    const uint32_t un = static_cast<uint32_t>(N);
    const int nq4 = (N + 3) >> 2;
    for (int j = wave; j < 2 * nq4; j += 4) {
        const bool is_q = j >= nq4;
        const uint32_t lr = static_cast<uint32_t>(lane) >> 4;
        const uint32_t r = 4u * j + lr;
        const uint32_t n = 4u * (is_q ? j - nq4 : j) + lr;
        const uint32_t c = (static_cast<uint32_t>(lane) & 15u) ^ (r & 15u);
        dma_x4(is_q ? Qh : Kh, (n < un ? n : 0u) * row_bytes + 16u * c, lds + 1024u * j);
    }
}

template <int NKT>
struct LargePrefetch {
    uint2 vraw[NKT];          // v of node 16 kt + lane % 16, rows v0..v0+3 (bf16)
    int par;                  // parent of node `lane` (tree walk layout)
    float alpha, beta;        // gates of node `lane`
};

template <int NKT>
__device__ __forceinline__ void large_prefetch(LargePrefetch<NKT>& pf, const uint16_t* V,
                                               const float* alpha, const float* beta,
                                               const int32_t* parent, int H, int N, int bh,
                                               int part, int wave, int lane) {
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;
    const uint32_t col = static_cast<uint32_t>(lane) & 15u;
    const uint32_t node_stride = static_cast<uint32_t>(H) * D;
    const uint16_t* Vh = V + (node0 * H + h) * D + part * kSmallRows + 16 * wave;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
        const uint32_t t = 16u * kt + col;
        pf.vraw[kt] = make_uint2(0u, 0u);
        if (t < static_cast<uint32_t>(N))
            pf.vraw[kt] = *reinterpret_cast<const uint2*>(Vh + (t * node_stride + 4u * (lane >> 4)));
    }
    pf.par = -1;
    pf.alpha = 1.0f;
    pf.beta = 0.0f;
    if (lane < N) {
        const size_t nh = (node0 + lane) * H + h;
        pf.par = parent[node0 + lane];
        pf.alpha = alpha[nh];
        pf.beta = beta[nh];
    }
}

// Whole half-rows of one item out of the U exchange (per wave w: [16 NKT nodes][16 values
// of rows 16w..16w+15 of the item's 64]) to a [nodes][H][D] fp32 array at dst (the head's
// node-0 row): wave w writes nodes 4 NKT w .. 4 NKT w + 4 NKT - 1, four 256-byte half-rows
// per store, lane l taking values 4 (l % 16)..+3 of the item's half from wave (l % 16) / 4's
// area.  Nodes past N get an offset past the buffer range and are dropped.  NKT stores per
// wave, with the streaming hint.
template <int NKT>
__device__ __forceinline__ void large_store_rows(float* dst, const float* Ub, int H, int N,
                                                 int part, int wave, int lane) {
    const uint32_t span = static_cast<uint32_t>(((N - 1) * H + 1) * D * sizeof(float));
    const int c = lane & 15;
#pragma unroll
    for (int i = 0; i < NKT; ++i) {
        const int t = 4 * NKT * wave + 4 * i + (lane >> 4);
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(
            Ub + (c >> 2) * (16 * NKT * 16) + t * 16 + 4 * (c & 3));
        const uint32_t off = t < N ? static_cast<uint32_t>((t * H * D + part * kSmallRows + 4 * c) * sizeof(float))
                                   : span;
        __builtin_amdgcn_raw_buffer_store_b128(
            x, __builtin_amdgcn_make_buffer_rsrc(dst, 0, span, kRawBufferFlags), off, 0, kStreamAux);
    }
}

template <int NKT>
__global__ __launch_bounds__(kSmallThreads)
__attribute__((amdgpu_waves_per_eu(3)))
void verify_large_kernel(
    const float* __restrict__ S0, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const float* __restrict__ alpha,
    const float* __restrict__ beta, const int32_t* __restrict__ parent, int H, int N, int BH,
    float* __restrict__ O, float* __restrict__ U, float* __restrict__ gamma,
    uint64_t* __restrict__ anc_out, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ status)
{
    using Lo = LargeLayout<NKT>;
    constexpr int NCT = 2 * NKT;
    constexpr int kCols = Lo::kCols;
    extern __shared__ __align__(16) float lds[];
    float* G = lds + Lo::kS0;                       // G[m][n], n: keys 0..N-1, queries 16NKT+t
    const char* ldsb = reinterpret_cast<const char*>(lds);
    const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    const int nq4 = (N + 3) >> 2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int grp = lane >> 4;
    static_assert(NKT == 2, "33 to 64 nodes run verify_head_kernel");
    float* Us = lds + Lo::kS0 + Lo::kG + wave * (16 * NKT * 16);   // this wave's U scratch
    const int grid = gridDim.x;
    const int slot = blockIdx.x;

    int bh, part;
    small_item(0, slot, grid, bh, part);
    if (bh >= BH) return;
    LargePrefetch<NKT> pf;
    small_issue_s0<false>(S0, lds, bh, part, wave, lane);
    large_prefetch<NKT>(pf, V, alpha, beta, parent, H, N, bh, part, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) asm volatile("" ::"v"(pf.vraw[kt]));
    asm volatile("" ::"v"(pf.par), "v"(pf.alpha), "v"(pf.beta));

    for (int round = 0;; ) {
        const int b = bh / H;
        const int h = bh - b * H;
        const size_t node0 = static_cast<size_t>(b) * N;

        uint2 vraw[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) vraw[kt] = pf.vraw[kt];
        const int my_par = pf.par;
        const float my_alpha = pf.alpha;
        const float my_beta = pf.beta;

        // this item's rows and inputs have landed once only the previous item's stores
        // (2 NKT, issued last) may still be in flight
        __builtin_amdgcn_s_waitcnt(Lo::kWait);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) asm volatile("" ::"v"(vraw[kt]));
        asm volatile("" ::"v"(my_par), "v"(my_alpha), "v"(my_beta));
        lds_barrier();

        // ---- tree walk, lane = node (every wave)
        uint64_t anc_l;
        float g_l, rg_l;
        {
            NodeInfo ni;
            {
                int p = my_par;
                const bool bad = lane < N && (p < -1 || p >= lane);
                if (bad) p = -1;
                uint64_t am = lane < N ? (1ull << lane) : 0ull;
                float g = lane < N ? my_alpha : 1.0f;
                int j = p;
                for (int r = 0; (1 << r) < N; ++r) {    // ceil(log2 N) rounds: depth <= N
                    const int src = j < 0 ? lane : j;
                    const uint64_t aj = shfl_u64(am, src);
                    const float gj = __shfl(g, src);
                    const int jj = __shfl(j, src);
                    if (j >= 0) { am |= aj; g *= gj; j = jj; }
                }
                ni.anc = am; ni.g = g; ni.depth = __popcll(am); ni.bad = bad;
            }
            anc_l = ni.anc;
            g_l = ni.g;
            rg_l = 1.0f / ni.g;
            if (wave == 0 && lane < N && part == 0) {
                if (ni.bad) report(status, TREEWY_ETREE);
                gamma[(node0 + lane) * H + h] = ni.g;
                if (h == 0) {
                    if (anc_out) anc_out[node0 + lane] = ni.anc;
                    if (depth_out) depth_out[node0 + lane] = ni.depth;
                }
            }
        }

        // ---- MFMA operands of this wave's 16 rows
        bf16x8_t ahi[4], alo[4];
        {
            const int r = 16 * wave + col;
            const float* rowp = lds + r * D;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int c0 = 2 * grp + 8 * ks;
                split_hi_lo(*reinterpret_cast<const f32x4_t*>(rowp + 4 * (c0 ^ (r & 15))),
                            *reinterpret_cast<const f32x4_t*>(rowp + 4 * ((c0 + 1) ^ (r & 15))),
                            ahi[ks], alo[ks]);
            }
        }
        lds_barrier();                              // rows read: the buffer may be refilled
        ++round;
        int bh_n, part_n;
        small_item(round, slot, grid, bh_n, part_n);
        const bool more = bh_n < BH;

        // the item's key and query rows go into the S-row area, free from here until the next
        // item's rows are requested (after the contractions)
        constexpr uint32_t kq_off = 0u;
        large_issue_kq(Q, K, H, N, bh, wave, lane, lds_addr);
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        float* Gx = G;

        // ---- contractions and Gram rows 16w..16w+15 (waves with keys there)
        const bool has_gram = wave < NKT && 16 * wave < N;
        bf16x8_t ka[4];
        {
            const uint32_t m = 16u * wave + col;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                u32x4_t w = {0u, 0u, 0u, 0u};
                if (has_gram && m < static_cast<uint32_t>(N))
                    w = *reinterpret_cast<const u32x4_t*>(
                        ldsb + kq_off + 256 * m + 16 * ((4 * ks + grp) ^ (m & 15)));
                ka[ks] = __builtin_bit_cast(bf16x8_t, w);
            }
        }
        f32x4_t acc[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            const uint32_t n = 16u * (c % NKT) + col;          // node of this column
            const bool is_q = c >= NKT;
            const bool live = n < static_cast<uint32_t>(N);
            const uint32_t r = is_q ? 4u * nq4 + n : n;            // staged row
            bf16x8_t bv[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                u32x4_t w = {0u, 0u, 0u, 0u};
                if (live)
                    w = *reinterpret_cast<const u32x4_t*>(
                        ldsb + kq_off + 256 * r + 16 * ((4u * ks + grp) ^ (r & 15u)));
                bv[ks] = __builtin_bit_cast(bf16x8_t, w);
            }
            acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            f32x4_t gacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[ks], bv[ks], acc[c], 0, 0, 0);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[ks], bv[ks], acc[c], 0, 0, 0);
                if (has_gram)
                    gacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], bv[ks], gacc, 0, 0, 0);
            }
            if (has_gram) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Gx[(16 * wave + 4 * grp + e) * kCols + 16 * c + col] = gacc[e];
            }
        }
        // the next item's rows only now: the key and query rows sit in the S-row area until
        // every wave is past the contractions
        lds_barrier();                              // G visible to every wave; inputs read
        if (more) {
            issue_s_pairs<false>(S0, lds_addr, bh_n, part_n, 0, 2, wave, lane);   // half the rows
            large_prefetch<NKT>(pf, V, alpha, beta, parent, H, N, bh_n, part_n, wave, lane);
        }

        // ---- per lane: nodes t = 16 kt + col, rows v0..v0+3
        float Uv[NKT][4], Ov[NKT][4];
        uint64_t mrem[NKT];
        float gt[NKT], bgt[NKT];
        int tn[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            const int t = 16 * kt + col;
            tn[kt] = t;
            const bool ok = t < N;
            const uint64_t a_t = shfl_u64(anc_l, t);
            const float g_t = ok ? __shfl(g_l, t) : 0.f;
            const float b_t = ok ? __shfl(my_beta, t) : 0.f;
            gt[kt] = g_t;
            bgt[kt] = b_t * g_t;
            mrem[kt] = ok ? (a_t & ~(1ull << t)) : 0ull;
            const float vv[4] = {__uint_as_float(vraw[kt].x << 16), __uint_as_float(vraw[kt].x & 0xffff0000u),
                                 __uint_as_float(vraw[kt].y << 16), __uint_as_float(vraw[kt].y & 0xffff0000u)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Uv[kt][e] = b_t * vv[e] - bgt[kt] * acc[kt][e];
                Ov[kt][e] = g_t * acc[NKT + kt][e];
            }
            *reinterpret_cast<f32x4_t*>(Us + t * 16 + 4 * grp) =
                f32x4_t{Uv[kt][0], Uv[kt][1], Uv[kt][2], Uv[kt][3]};
        }
        // ancestor walk: step d folds in every node's depth-d ancestor (final since step d - 1).
        // The coefficients of a step (ancestor gates by lane permute, Gram entries) do not
        // depend on U, so those of step d + 1 are requested while step d's U rows are read.
        float cs[NKT], cw[NKT];
        int asel[NKT];
        auto coeffs = [&](float (&cs_)[NKT], float (&cw_)[NKT], int (&as_)[NKT]) {
            float rgsrc[NKT];
            bool hasa[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                hasa[kt] = mrem[kt] != 0ull;
                as_[kt] = hasa[kt] ? __ffsll(static_cast<unsigned long long>(mrem[kt])) - 1 : tn[kt] & 63;
                mrem[kt] &= mrem[kt] - 1;
                rgsrc[kt] = __shfl(rg_l, as_[kt]);
            }
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const int a = as_[kt];
                const int t = tn[kt];
                cs_[kt] = hasa[kt] ? bgt[kt] * rgsrc[kt] * Gx[t * kCols + a] : 0.f;
                cw_[kt] = hasa[kt] ? gt[kt] * rgsrc[kt] * Gx[a * kCols + 16 * NKT + t] : 0.f;
            }
        };
        auto pending = [&]() {
            bool any = false;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) any |= mrem[kt] != 0ull;
            return __any(any) != 0;
        };
        bool step = pending();
        if (step) coeffs(cs, cw, asel);
        while (step) {
            f32x4_t x[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                x[kt] = *reinterpret_cast<const f32x4_t*>(Us + asel[kt] * 16 + 4 * grp);
            float cs_n[NKT], cw_n[NKT];
            int as_n[NKT];
            step = pending();
            if (step) coeffs(cs_n, cw_n, as_n);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Uv[kt][e] -= cs[kt] * x[kt][e];
                    Ov[kt][e] += cw[kt] * x[kt][e];
                }
                *reinterpret_cast<f32x4_t*>(Us + tn[kt] * 16 + 4 * grp) =
                    f32x4_t{Uv[kt][0], Uv[kt][1], Uv[kt][2], Uv[kt][3]};
            }
            if (step) {
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    cs[kt] = cs_n[kt];
                    cw[kt] = cw_n[kt];
                    asel[kt] = as_n[kt];
                }
            }
        }
        if (more)                                   // the other half of the next item's rows
            issue_s_pairs<false>(S0, lds_addr, bh_n, part_n, 4, 2, wave, lane);
        // the node's own term; then O and U out as whole half-rows (the item's 64 values of
        // a node, 256 bytes), assembled in the U exchange: a wave's own stores would cover
        // only 64 bytes of each
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            const int t = tn[kt];
            const float cw = t < N ? Gx[t * kCols + 16 * NKT + t] : 0.f;   // the node itself
#pragma unroll
            for (int e = 0; e < 4; ++e) Ov[kt][e] += cw * Uv[kt][e];
        }
        const size_t row0 = (node0 * H + h) * D;
        const float* Ub = lds + Lo::kS0 + Lo::kG;
        lds_barrier();                              // every wave's U rows in its exchange area
        large_store_rows<NKT>(U + row0, Ub, H, N, part, wave, lane);
        lds_barrier();                              // ... and read
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
            *reinterpret_cast<f32x4_t*>(Us + tn[kt] * 16 + 4 * grp) =
                f32x4_t{Ov[kt][0], Ov[kt][1], Ov[kt][2], Ov[kt][3]};
        lds_barrier();                              // O rows in the exchange
        large_store_rows<NKT>(O + row0, Ub, H, N, part, wave, lane);
        if (!more) break;
        bh = bh_n;
        part = part_n;
    }
}

// ---------------------------------------------------------------------------------------
// One head per item: the fused and deferred steps on 17 to 64 nodes, the plain verify on 33
// to 64 (NKT = 2 node tiles up to 32 nodes, 3 up to 48, 4 above).
//
// A workgroup of eight waves takes whole heads (all 128 value rows; wave w owns rows
// 16w..16w+15), one workgroup per CU, and walks a run of consecutive heads, so the heads
// of one sequence follow one another: its tree bookkeeping (ancestor masks, the
// pointer-jumping targets) and its previous accepted path are derived once per run, and
// each head only forms its own gates g_t as products over the cached jump targets.
//
// Every input of head i + 1 is requested during head i, by direct HBM -> LDS transfers
// into areas that head i no longer needs: its S rows once head i's rows are in registers
// (after the commit and the operand split), in four quarters spread over head i (after the
// split, after the Gram tiles, after the contractions, with the other inputs; see
// issue_s_pairs; the plain verify in two halves), the previous step's path rows for its commit with the first quarter, its
// key, query and value rows, parents and gates once head i's contractions are done.  So a
// head finds its inputs in place, and no register carries them across a head.
//
// The key/query rows are staged once per head for all eight waves.  The Gram entries the
// solve uses (key . key below the diagonal, key . query above it) are formed on the matrix
// cores by 16 x 16 tiles: key rows 16 rt.. have NKT + 1 tiles, dealt to the 8 / NKT waves
// of that row tile.  This runs after the next head's S rows are requested (it needs only
// the key/query rows and the gates), so that transfer overlaps it.  The entries go, already
// scaled, into compact coefficient tables indexed by the ancestor's depth,
//   C[d-1][t] = b_t (g_t / g_a) (k_t . k_a)     (a the depth-d ancestor of t, strict),
//   W[d-1][t] = (g_t / g_a) (k_a . q_t)         (a the depth-d ancestor-or-self of t),
// which step d of the ancestor walk reads together with the ancestors' U rows: one LDS
// round trip per step.  Ancestors deeper than the tables (kHeadSlots) get their
// coefficients from the key and query rows in memory during the walk instead.

constexpr int kHeadWaves = 8;
constexpr int kHeadThreads = 64 * kHeadWaves;
constexpr int kHeadSlots = 16;                 // ancestor depths with staged coefficients
constexpr int kHeadListPer = 5;                // ancestors per packed list word (6 bits each)
constexpr int kHeadListWords = 3;              // list words per node: depths 1..15
static_assert(kHeadListPer * kHeadListWords < kHeadSlots, "listed depths have table slots");
// s_waitcnt operand: vmcnt <= 8, no other wait
constexpr int kVmcnt8 = 8 | (7 << 4) | (15 << 8);

// LDS of one head workgroup (byte offsets):
//   S   S rows [128][128] fp32 (16-byte chunk c of row r at chunk c ^ (r % 16))
//   KQ  key rows 0 .. 16 NKT - 1, query rows 16 NKT .. 32 NKT - 1 (256 B, the same
//       swizzle; rows of nodes past N are never read into a result that is used)
//   U   per wave the U exchange [16 NKT nodes][16 rows] fp32; after the walk it assembles
//       whole U rows, then whole O rows, for the stores
//   C,W coefficient tables [kHeadSlots][16 NKT] fp32
//   V   value rows [16 NKT][128] bf16 (the same swizzle)
//   PU, PK, PG  the previous step's commit terms of one chunk (kPath of them: U_prev or
//       logged u~ rows 512 B, K_prev or logged key rows 256 B), the path's gammas [64].
//       Sixteen terms per chunk up to 48 nodes, eight at 49-64 (where the LDS is full)
//   SM  parents, alphas, betas of the head (64 words each)
//   PI, PA  the previous tree (64 words) and accepted node (one word, repeated) of a later
//       head's sequence
//   LN, LS  deferred commit: the log length of that sequence and the next head's log scale
//       (one word each, repeated)
//   O   (NKT = 2 only, where the LDS has room) an O exchange beside the U one, so that the
//       O rows are assembled while the U rows are and both leave after one barrier
template <int NKT>
struct HeadLds {
    static constexpr int kNodes = 16 * NKT;
    static constexpr int kPath = NKT <= 3 ? 16 : 8;       // commit terms staged per chunk
    static constexpr uint32_t kS = 0;
    static constexpr uint32_t kKQ = kS + D * D * 4u;
    static constexpr uint32_t kU = kKQ + 2u * kNodes * 256u;
    static constexpr uint32_t kC = kU + kHeadWaves * kNodes * 16u * 4u;
    static constexpr uint32_t kW = kC + kHeadSlots * kNodes * 4u;
    static constexpr uint32_t kV = kW + kHeadSlots * kNodes * 4u;
    static constexpr uint32_t kPU = kV + kNodes * 256u;
    static constexpr uint32_t kPK = kPU + kPath * D * 4u;
    static constexpr uint32_t kPG = kPK + kPath * D * 2u;
    static constexpr uint32_t kSM = kPG + 256u;
    static constexpr uint32_t kPI = kSM + 768u;
    static constexpr uint32_t kPA = kPI + 256u;
    static constexpr uint32_t kLN = kPA + 256u;
    static constexpr uint32_t kLS = kLN + 256u;
    static constexpr bool kOwnO = NKT == 2;
    static constexpr uint32_t kO = kLS + 256u;
    static constexpr uint32_t kBytes = kO + (kOwnO ? kHeadWaves * kNodes * 16u * 4u : 0u);
    static_assert(kBytes <= 160u * 1024u, "one workgroup per CU");
    // s_waitcnt operand: vmcnt <= 2 NKT (the previous head's NKT O and NKT U row stores per
    // wave), no other wait
    static constexpr int kWait = (2 * NKT) | (7 << 4) | (15 << 8);
};


// A head's key, query and value rows, parents, alphas and betas -> LDS (layout above): per
// four nodes one transfer of key rows, one of query rows and one of value rows, then three
// gathers, dealt round-robin to waves w0..7.  Lanes past the last node load node 0.  With
// `with_parents` false the parents are left out (already requested).
template <int NKT>
__device__ __forceinline__ void head_issue_inputs(const uint16_t* Q, const uint16_t* K,
                                                  const uint16_t* V, const float* alpha,
                                                  const float* beta, const int32_t* parent,
                                                  int H, int N, int bh, int wave, int lane,
                                                  uint32_t lds, int w0 = 0,
                                                  bool with_parents = true) {
    using L = HeadLds<NKT>;
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * N;
    const uint32_t row_bytes = static_cast<uint32_t>(H) * D * 2;
    const size_t hoff = (node0 * H + h) * D;
    const uint32_t un = static_cast<uint32_t>(N);
    const uint32_t ln = static_cast<uint32_t>(lane) < un ? static_cast<uint32_t>(lane) : 0u;
    const int nq4 = (N + 3) >> 2;
    const int jobs = 3 * nq4 + 3;
    if (wave < w0) return;
    for (int j = wave - w0; j < jobs; j += kHeadWaves - w0) {
        if (j < 3 * nq4) {
            const int kind = j / nq4;                    // 0 keys, 1 queries, 2 values
            const int jj = j - kind * nq4;
            const uint32_t lr = static_cast<uint32_t>(lane) >> 4;
            const uint32_t n = 4u * jj + lr;             // node
            const uint32_t r = kind == 1 ? static_cast<uint32_t>(L::kNodes) + n : n;   // row in its area
            const uint32_t c = (static_cast<uint32_t>(lane) & 15u) ^ (r & 15u);
            const uint16_t* src = (kind == 0 ? K : kind == 1 ? Q : V) + hoff;
            const uint32_t dst = kind == 2 ? L::kV + 1024u * jj
                                           : L::kKQ + 256u * (kind * L::kNodes) + 1024u * jj;
            dma_x4(src, (n < un ? n : 0u) * row_bytes + 16u * c, lds + dst);
        } else if (j == 3 * nq4) {
            if (with_parents) dma_x1(parent + node0, 4u * ln, lds + L::kSM);
        } else if (j == 3 * nq4 + 1) {
            dma_x1(alpha + node0 * H + h, 4u * ln * static_cast<uint32_t>(H), lds + L::kSM + 256u);
        } else {
            dma_x1(beta + node0 * H + h, 4u * ln * static_cast<uint32_t>(H), lds + L::kSM + 512u);
        }
    }
}

// The previous tree and accepted node of head bh's sequence -> LDS (PI, PA), and with the
// deferred commit its log length (LN), by one wave.
template <int NKT>
__device__ __forceinline__ void head_issue_prev_tree(const CommitIn& c, int bh, int H, int lane,
                                                     uint32_t lds, const int32_t* len_in = nullptr) {
    using L = HeadLds<NKT>;
    const int b = bh / H;
    const uint32_t n = static_cast<uint32_t>(lane) < static_cast<uint32_t>(c.Np)
                           ? static_cast<uint32_t>(lane) : 0u;
    dma_x1(c.parent + static_cast<size_t>(b) * c.Np, 4u * n, lds + L::kPI);
    dma_x1(c.accepted + b, 0u, lds + L::kPA);
    if (len_in) dma_x1(len_in + b, 0u, lds + L::kLN);
}

// Path rows P c .. P c + P - 1 of a head -> LDS (P = kPath): U_prev rows (two per
// transfer), K_prev rows (four per transfer), and with the first chunk the gammas of the
// whole path (one gather, lane = path position).  Slots past the path repeat its first node.
template <int NKT>
__device__ __forceinline__ void head_issue_path(const CommitIn& c, const PathInfo& pi, int chunk,
                                                int bh, int H, int wave, int lane, uint32_t lds) {
    using L = HeadLds<NKT>;
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * c.Np;
    const int cnt = pi.depth - L::kPath * chunk < L::kPath ? pi.depth - L::kPath * chunk : L::kPath;
    const int nu = (cnt + 1) >> 1;
    const int nk = (cnt + 3) >> 2;
    const int jobs = nu + nk + (chunk == 0 ? 1 : 0);
    const float* Uh = c.U + (node0 * H + h) * D;
    const uint16_t* Kh = c.K + (node0 * H + h) * D;
    for (int j = wave; j < jobs; j += kHeadWaves) {
        if (j < nu) {
            const int q = 2 * j + (lane >> 5);
            const uint32_t n = static_cast<uint32_t>(__shfl(pi.pn, L::kPath * chunk + (q < cnt ? q : 0)));
            dma_x4(Uh, n * static_cast<uint32_t>(H) * (D * 4u) + 16u * (static_cast<uint32_t>(lane) & 31u),
                   lds + L::kPU + 1024u * j);
        } else if (j < nu + nk) {
            const int jj = j - nu;
            const int q = 4 * jj + (lane >> 4);
            const uint32_t n = static_cast<uint32_t>(__shfl(pi.pn, L::kPath * chunk + (q < cnt ? q : 0)));
            dma_x4(Kh, n * static_cast<uint32_t>(H) * (D * 2u) +
                           16u * ((static_cast<uint32_t>(lane) & 15u) ^ head_pk_swizzle(q)),
                   lds + L::kPK + 1024u * jj);
        } else {
            const int n = __shfl(pi.pn, lane < pi.depth ? lane : 0);
            dma_gather_x1(c.gamma + (node0 + n) * H + h, lds + L::kPG);
        }
    }
}

// The log length of the sequence whose previous tree sits in LDS (LN), clamped to
// [0, Lmax]; a length outside is reported (TREEWY_ELOG) by the reporting lane.
template <int NKT>
__device__ __forceinline__ int head_log_len(const char* ldsb, int Lmax, bool reporter,
                                            int32_t* status) {
    const int raw = __builtin_amdgcn_readfirstlane(
        reinterpret_cast<const int*>(ldsb + HeadLds<NKT>::kLN)[0]);
    const int len = log_len(raw, Lmax);
    if (raw != len && reporter) report(status, TREEWY_ELOG);
    return len;
}

// The deferred commit's rank-one terms of a head, chunk c (slots P c .. P c + P - 1,
// P = kPath) -> LDS: slot s < len is log term s (u~ row from the log, key row from the log),
// slot s >= len is path node s - len (U_prev row, K_prev row), in the path slots (PU, PK;
// every row by a per-lane gather, since the two sources are separate arrays).  With the
// first chunk also the path's gammas (PG) and the head's log scale (LS).  Slots past the
// terms repeat slot 0.
template <int NKT>
__device__ __forceinline__ void head_issue_terms(const CommitIn& c, const DeferLog& dl,
                                                 const PathInfo& pi, int len, int chunk, int bh,
                                                 int H, int wave, int lane, uint32_t lds) {
    using L = HeadLds<NKT>;
    const int b = bh / H;
    const int h = bh - b * H;
    const size_t node0 = static_cast<size_t>(b) * c.Np;
    const int rem = len + pi.depth - L::kPath * chunk;
    const int cnt = rem < L::kPath ? rem : L::kPath;
    const int nu = cnt > 0 ? (cnt + 1) >> 1 : 0;
    const int nk = cnt > 0 ? (cnt + 3) >> 2 : 0;
    const int jobs = nu + nk + (chunk == 0 ? 2 : 0);
    const size_t lrow0 = static_cast<size_t>(bh) * dl.Lmax;
    for (int j = wave; j < jobs; j += kHeadWaves) {
        if (j < nu + nk) {
            const bool is_k = j >= nu;
            const int jj = is_k ? j - nu : j;
            const int q = is_k ? 4 * jj + (lane >> 4) : 2 * jj + (lane >> 5);
            const int sl = L::kPath * chunk + (q < cnt ? q : 0);
            const int pq = sl - len;                       // path position (slot >= len)
            const int n = __shfl(pi.pn, pq >= 0 ? pq : 0);
            if (is_k) {
                const uint16_t* src = sl < len ? dl.K + (lrow0 + sl) * D
                                               : c.K + ((node0 + n) * H + h) * D;
                dma_gather_x4(src + 8 * ((static_cast<uint32_t>(lane) & 15u) ^ head_pk_swizzle(q)),
                              lds + L::kPK + 1024u * jj);
            } else {
                const float* src = sl < len ? dl.U + (lrow0 + sl) * D
                                            : c.U + ((node0 + n) * H + h) * D;
                dma_gather_x4(src + 4 * (lane & 31), lds + L::kPU + 1024u * jj);
            }
        } else if (j == nu + nk) {
            const int n = __shfl(pi.pn, lane < pi.depth ? lane : 0);
            dma_gather_x1(c.gamma + (node0 + n) * H + h, lds + L::kPG);
        } else {
            dma_x1(dl.scale_in + bh, 0u, lds + L::kLS);
        }
    }
}

// One staged chunk of commit terms applied to this wave's 16 rows of S in LDS, on the matrix
// cores (apply_terms): U rows of 512 bytes in PU, key rows in PK with 16-byte chunks swizzled
// by head_pk_swizzle.
template <int NKT>
__device__ __forceinline__ void head_apply_terms(float* lds, uint32_t lds_addr, int cnt,
                                                 const float (&coef)[4], float c0, int wave,
                                                 int lane) {
    using L = HeadLds<NKT>;
    apply_terms<D, true>(lds, lds_addr, cnt, coef, c0, L::kPU, L::kPK, L::kPath, wave, lane);
}

// This wave's 16 rows of S, final in LDS, to S in HBM as whole 512-byte rows (lane l: row
// 16w + 2i + l / 32, 16-byte chunk l % 32, i = 0..7), with the streaming hint (the state is
// read once and written once per step).  The rows were written by other lanes of this wave;
// a wave's LDS accesses complete in issue order.
template <int NKT>
__device__ __forceinline__ void head_store_state(const float* lds, float* S, int bh, int wave,
                                                 int lane) {
    const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
    const uint32_t ch = static_cast<uint32_t>(lane) & 31u;
    asm volatile("" ::: "memory");            // after the rows' last LDS writes
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t r = 16u * wave + 2u * i + hl;
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(lds + r * D + 4 * (ch ^ (r & 15u)));
        __builtin_nontemporal_store(
            x, reinterpret_cast<f32x4_t*>(S + (static_cast<size_t>(bh) * D + r) * D + 4 * ch));
    }
}

// The deferred commit on this wave's 16 rows of a head.  With the log read as len terms
// u~_j k_j^T and scale s, the committed state after this step is
//   S_a = gs (S + sum_j u~_j k_j^T) + sum over the path of a of (g_a / g_i) U_prev[i] k_i^T,
// gs = s g_a (paper §3 "Reconstruct on commit", Eq. 3, applied to the logged state), formed
// in LDS on the matrix cores (head_apply_terms) for this step's contractions.  When the path's terms fit in the log and in one
// chunk of slots (len + depth <= min(Lmax, kPath)) they are appended to the log as
// u~ = (g_a / g_i) U_prev[i] / gs (one wave per term: the 512-byte u~ row and the 256-byte
// key row) and S is not written; otherwise S_a goes to S as whole rows and the log is
// emptied.  The header after the step: scale 1 and length 0 when emptied, else gs and
// len + depth.  Called by every wave, with len + depth > 0.
template <int NKT>
__device__ __forceinline__ void head_commit_defer(float* lds, const PathInfo& cur, int len,
                                                  const CommitIn& cin, const DeferLog& dl,
                                                  int bh, int H, int wave, int lane,
                                                  uint32_t lds_addr) {
    using L = HeadLds<NKT>;
    const char* ldsb = reinterpret_cast<const char*>(lds);
    const float* PG = reinterpret_cast<const float*>(ldsb + L::kPG);
    const float* PU = reinterpret_cast<const float*>(ldsb + L::kPU);
    const char* PK = ldsb + L::kPK;
    const float gin = reinterpret_cast<const float*>(ldsb + L::kLS)[0];
    const float ga = cur.depth > 0 ? PG[cur.depth - 1] : 1.0f;
    const float gs = gin * ga;
    const int total = len + cur.depth;
    const int keep = dl.Lmax < L::kPath ? dl.Lmax : L::kPath;
    const bool flush = total > keep;
    const int g = lane >> 4;
    const int nchunk = (total + L::kPath - 1) / L::kPath;
    for (int ci = 0; ci < nchunk; ++ci) {
        const int q0 = ci * L::kPath;
        if (ci > 0) {
            lds_barrier();
            head_issue_terms<NKT>(cin, dl, cur, len, ci, bh, H, wave, lane, lds_addr);
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier();
        }
        const int rem = total - q0;
        const int cnt = rem < L::kPath ? rem : L::kPath;
        // log terms carry the new scale; path term i carries g_a / g_i
        float coef[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int sl = q0 + 4 * g + t;
            const int pq = sl - len;
            coef[t] = sl < len ? gs : ga * __builtin_amdgcn_rcpf(PG[pq >= 0 && pq < 64 ? pq : 0]);
        }
        head_apply_terms<NKT>(lds, lds_addr, cnt, coef, ci == 0 ? gs : 1.0f, wave, lane);
    }
    if (!flush) {
        // every term sits in the first chunk's slots: path node q is slot len + q
        const size_t lrow0 = static_cast<size_t>(bh) * dl.Lmax + len;
        const float rgs = 1.0f / gs;
        for (int q = wave; q < cur.depth; q += kHeadWaves) {
            const int sl = len + q;
            if (lane < 32) {
                const float cq = (ga / PG[q]) * rgs;
                const f32x4_t u = *reinterpret_cast<const f32x4_t*>(PU + sl * D + 4 * lane);
                *reinterpret_cast<f32x4_t*>(dl.U + (lrow0 + q) * D + 4 * lane) = cq * u;
            } else if (lane < 48) {
                const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(
                    PK + sl * 256 + 16 * ((static_cast<uint32_t>(lane) - 32u) ^ head_pk_swizzle(sl)));
                *reinterpret_cast<u32x4_t*>(dl.K + (lrow0 + q) * D + 8 * (lane - 32)) = kv;
            }
        }
    }
    if (wave == 0 && lane == 0) {
        const int b = bh / H;
        dl.scale_out[bh] = flush ? 1.0f : gs;
        if (bh - b * H == 0) dl.len_out[b] = flush ? 0 : total;
    }
    if (flush) head_store_state<NKT>(lds, cin.S, bh, wave, lane);
}

// The previous step's commit on this wave's 16 rows of a head, in LDS: S_a = g_a S + sum
// over the path of a of (g_a / g_i) U_prev[i] k_i^T (paper §3 "Reconstruct on commit",
// Eq. 3), on the matrix cores (head_apply_terms; paths of up to cin.short_path nodes on the
// vector ALUs), written back to LDS for this step's contractions and to S as whole 512-byte
// rows.
// The first kPath path rows and all the path's gammas are in LDS; a longer path fetches the
// rest chunk by chunk, with blocking waits.  Every wave calls it (the path is the same for
// the whole workgroup).
template <int NKT>
__device__ __forceinline__ void head_commit_rows(float* lds, const PathInfo& cur, const CommitIn& cin,
                                                 int bh, int H, int wave, int lane,
                                                 uint32_t lds_addr) {
    using L = HeadLds<NKT>;
    const char* ldsb = reinterpret_cast<const char*>(lds);
    const float* PG = reinterpret_cast<const float*>(ldsb + L::kPG);
    const float ga = PG[cur.depth - 1];
    if (cur.depth <= cin.short_path) {
        // a short path (cin.short_path <= 8, one staged chunk): the terms on the vector ALUs,
        // in the rows' arrival layout (lane l: row 16w + 2i + l / 32, 16-byte chunk l % 32,
        // i = 0..7), which has less latency than the matrix-core form for so few terms
        const float* PU = reinterpret_cast<const float*>(ldsb + L::kPU);
        const char* PK = ldsb + L::kPK;
        const uint32_t hl = static_cast<uint32_t>(lane) >> 5;
        const uint32_t ch = static_cast<uint32_t>(lane) & 31u;   // values 4 ch .. 4 ch + 3
        f32x4_t x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t r = 16u * wave + 2u * i + hl;
            x[i] = ga * *reinterpret_cast<const f32x4_t*>(lds + r * D + 4 * (ch ^ (r & 15u)));
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q >= cur.depth) break;
            const float cq = ga * __builtin_amdgcn_rcpf(PG[q]);
            const uint2 kw = *reinterpret_cast<const uint2*>(
                PK + q * 256 + 16 * ((ch >> 1) ^ head_pk_swizzle(q)) + 8 * (ch & 1u));
            const f32x4_t kv = {__uint_as_float(kw.x << 16), __uint_as_float(kw.x & 0xffff0000u),
                                __uint_as_float(kw.y << 16), __uint_as_float(kw.y & 0xffff0000u)};
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] += (cq * PU[q * D + 16 * wave + 2 * i + hl]) * kv;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t r = 16u * wave + 2u * i + hl;
            *reinterpret_cast<f32x4_t*>(lds + r * D + 4 * (ch ^ (r & 15u))) = x[i];
            __builtin_nontemporal_store(
                x[i], reinterpret_cast<f32x4_t*>(cin.S + (static_cast<size_t>(bh) * D + r) * D + 4 * ch));
        }
        return;
    }
    const int g = lane >> 4;
    const int nchunk = (cur.depth + L::kPath - 1) / L::kPath;
    for (int ci = 0; ci < nchunk; ++ci) {
        const int q0 = ci * L::kPath;
        if (ci > 0) {
            lds_barrier();
            head_issue_path<NKT>(cin, cur, ci, bh, H, wave, lane, lds_addr);
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier();
        }
        const int rem = cur.depth - q0;
        const int cnt = rem < L::kPath ? rem : L::kPath;
        float coef[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int q = q0 + 4 * g + t;
            coef[t] = ga * __builtin_amdgcn_rcpf(PG[q < 64 ? q : 0]);
        }
        head_apply_terms<NKT>(lds, lds_addr, cnt, coef, ci == 0 ? ga : 1.0f, wave, lane);
    }
    head_store_state<NKT>(lds, cin.S, bh, wave, lane);
}

// Whole node rows of one head out of the U exchange (per wave w: [node][16 values of rows
// 16w..16w+15]) to a [nodes][H][D] fp32 array at dst (the head's node-0 row): wave w writes
// nodes 2 NKT w .. 2 NKT w + 2 NKT - 1, two 512-byte rows per store, lane l taking values
// 4 (l % 32)..+3 of node 2 NKT w + 2i + l / 32 from wave (l % 32) / 4's area.  Nodes past N
// fall outside the buffer range and are dropped.  NKT stores per wave, with the streaming
// hint.
template <int NKT>
__device__ __forceinline__ void head_store_rows(float* dst, const char* ldsb, int H, int N,
                                                int wave, int lane, uint32_t area = HeadLds<NKT>::kU) {
    using L = HeadLds<NKT>;
    static_assert(L::kNodes == 2 * NKT * kHeadWaves, "2 NKT nodes per wave");
    const float* Ub = reinterpret_cast<const float*>(ldsb + area);
    const uint32_t span = static_cast<uint32_t>(((N - 1) * H + 1) * D * sizeof(float));
    const int c = lane & 31;
#pragma unroll
    for (int i = 0; i < NKT; ++i) {
        const int t = 2 * NKT * wave + 2 * i + (lane >> 5);
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(
            Ub + (c >> 2) * (L::kNodes * 16) + t * 16 + 4 * (c & 3));
        const uint32_t off = t < N ? static_cast<uint32_t>((t * H * D + 4 * c) * sizeof(float)) : span;
        __builtin_amdgcn_raw_buffer_store_b128(
            x, __builtin_amdgcn_make_buffer_rsrc(dst, 0, span, kRawBufferFlags), off, 0, kStreamAux);
    }
}

// Part of the dot product of two bf16 rows of 128 elements: elements 32 grp .. 32 grp + 31,
// then summed over the four lanes col, col + 16, col + 32, col + 48.  Called by all lanes.
// A sequence's tree as each lane of the head kernel keeps it (lane = node): its ancestor
// mask, its pointer-jump targets, the tree's depth and jump rounds, and for the lane's nodes
// t = 16 kt + lane % 16 their depth and strict ancestors in depth order (packed 6 bits each,
// 0 past the list).
template <int NKT>
struct HeadTree {
    uint64_t anc_l;
    int jp[6];
    int maxd, grounds;
    int dtk[NKT];
    uint32_t alist[NKT][kHeadListWords];
};

// Derive it from the parents (lane = node; -1 past N); a malformed parent is reported and
// taken as a root.
template <int NKT>
__device__ __forceinline__ void head_tree(int my_par, int N, int lane, int32_t* status,
                                          HeadTree<NKT>& tr) {
    const int col = lane & 15;
    int p = my_par;
    const bool bad = lane < N && (p < -1 || p >= lane);
    if (bad) p = -1;
    uint64_t am = lane < N ? (1ull << lane) : 0ull;
    int j = p;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        tr.jp[r] = j;
        if ((1 << r) < N) {
            const int src = j < 0 ? lane : j;
            const uint64_t aj = shfl_u64(am, src);
            const int jj = __shfl(j, src);
            if (j >= 0) { am |= aj; j = jj; }
        }
    }
    tr.anc_l = am;
    if (bad) report(status, TREEWY_ETREE);
    int dm = __popcll(am);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dm = max(dm, __shfl_xor(dm, off));
    tr.maxd = __builtin_amdgcn_readfirstlane(dm);
    tr.grounds = 0;
    while ((1 << tr.grounds) < tr.maxd) ++tr.grounds;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
        const int t = 16 * kt + col;
        const uint64_t at0 = shfl_u64(am, t);
        const uint64_t at = t < N ? at0 : 0ull;
        tr.dtk[kt] = __popcll(at);
        uint64_t m = at & ~(1ull << t);
#pragma unroll
        for (int wd = 0; wd < kHeadListWords; ++wd) {
            uint32_t w = 0u;
#pragma unroll
            for (int i = 0; i < kHeadListPer; ++i) {
                const uint32_t x = m != 0ull ? static_cast<uint32_t>(__ffsll(static_cast<unsigned long long>(m)) - 1) : 0u;
                m &= m - 1ull;
                w |= x << (6 * i);
            }
            tr.alist[kt][wd] = w;
        }
    }
}

__device__ __forceinline__ float head_dot_bf16(const uint16_t* x, const uint16_t* y, int grp) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 a = *reinterpret_cast<const uint4*>(x + 32 * grp + 8 * j);
        const uint4 b = *reinterpret_cast<const uint4*>(y + 32 * grp + 8 * j);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            s += __uint_as_float(aw[k] << 16) * __uint_as_float(bw[k] << 16);
            s += __uint_as_float(aw[k] & 0xffff0000u) * __uint_as_float(bw[k] & 0xffff0000u);
        }
    }
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    return s;
}

template <int NKT, bool FUSED, bool DEFER = false>
__global__ __launch_bounds__(kHeadThreads)
void verify_head_kernel(
    const float* __restrict__ S0, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const float* __restrict__ alpha,
    const float* __restrict__ beta, const int32_t* __restrict__ parent, int H, int N, int BH,
    float* __restrict__ O, float* __restrict__ U, float* __restrict__ gamma,
    uint64_t* __restrict__ anc_out, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ status, CommitIn cin, DeferLog dlog)
{
    using L = HeadLds<NKT>;
    constexpr int NCT = 2 * NKT;
    constexpr int NN = L::kNodes;
    // the next head's S rows go out in four parts with the commit (fused), in two halves
    // without (after the split and after the contractions: measured 173 -> 170 us per
    // 64-node layer, where four parts suit the fused step)
    constexpr int kSParts = FUSED ? 4 : 2;
    extern __shared__ __align__(16) float lds[];
    char* ldsb = reinterpret_cast<char*>(lds);
    const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    float* Ct = reinterpret_cast<float*>(ldsb + L::kC);
    float* Wt = reinterpret_cast<float*>(ldsb + L::kW);

    const int tid = threadIdx.x;
    const int lane0 = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // this workgroup's heads: [lo, hi), consecutive
    const int G = gridDim.x;
    const int s = blockIdx.x;
    const int qh = BH / G;
    const int rh = BH - qh * G;
    const int lo = s * qh + (s < rh ? s : rh);
    const int hi = lo + qh + (s < rh ? 1 : 0);
    if (lo >= hi) return;

    // ---- prologue: wave 0 requests the first head's parents (and, fused, the previous tree
    // and accepted node of its sequence), then every wave its S rows and the other inputs
    // (waves 1-7); the sequence's tree (and, fused, the accepted path, whose rows are
    // requested next) is derived while those land.  Wave 0's eight S-row transfers are the
    // only ones it issues after its first ones.
    PathInfo pnext{0ull, 0, 0};
    int plen = 0;                             // deferred: the log length of pnext's sequence
    const int32_t* len_in = DEFER ? dlog.len_in : nullptr;
    if (wave == 0) {
        const uint32_t ln = static_cast<uint32_t>(lane0) < static_cast<uint32_t>(N)
                                ? static_cast<uint32_t>(lane0) : 0u;
        dma_x1(parent + static_cast<size_t>(lo / H) * N, 4u * ln, lds_addr + L::kSM);
        if constexpr (FUSED) head_issue_prev_tree<NKT>(cin, lo, H, lane0, lds_addr, len_in);
    }
    small_issue_s0<FUSED>(S0, lds, lo, 0, wave, lane0);
    head_issue_inputs<NKT>(Q, K, V, alpha, beta, parent, H, N, lo, wave, lane0, lds_addr, 1, false);
    if (wave == 0) __builtin_amdgcn_s_waitcnt(kVmcnt8);
    lds_barrier();
    int seq = lo / H;
    HeadTree<NKT> tr;
    head_tree<NKT>(lane0 < N ? reinterpret_cast<const int*>(ldsb + L::kSM)[lane0] : -1, N, lane0,
                   status, tr);
    if constexpr (FUSED) {
        const int pidx = lane0 < cin.Np ? reinterpret_cast<const int*>(ldsb + L::kPI)[lane0] : -1;
        const int pacc = reinterpret_cast<const int*>(ldsb + L::kPA)[0];
        pnext = fused_path(pidx, pacc, cin.Np, lane0, wave == 0 && lo % H == 0, status);
        if constexpr (DEFER)
            plen = head_log_len<NKT>(ldsb, dlog.Lmax, wave == 0 && lane0 == 0 && lo % H == 0, status);
        lds_barrier();                        // the previous tree read: refill
        if constexpr (DEFER)
            head_issue_terms<NKT>(cin, dlog, pnext, plen, 0, lo, H, wave, lane0, lds_addr);
        else if (pnext.depth > 0)
            head_issue_path<NKT>(cin, pnext, 0, lo, H, wave, lane0, lds_addr);
        if (lo + 1 < hi && wave == kHeadWaves - 1)
            head_issue_prev_tree<NKT>(cin, lo + 1, H, lane0, lds_addr, len_in);
    }
    __builtin_amdgcn_s_waitcnt(0);


    for (int bh = lo;; ) {
        const int b = bh / H;
        const int h = bh - b * H;
        const size_t node0 = static_cast<size_t>(b) * N;
        const bool more = bh + 1 < hi;
        // the lane index made opaque here, so that the many lane-dependent LDS addresses
        // below are formed inside each head instead of being held in registers for the
        // whole loop
        int lane = lane0;
        asm volatile("" : "+v"(lane));
        const int col = lane & 15;
        const int grp = lane >> 4;
        float* Us = reinterpret_cast<float*>(ldsb + L::kU) + wave * (NN * 16);

        // this head's inputs: everything was requested during the previous head (or the
        // prologue); only that head's O and U stores, issued last, may still be in flight
        __builtin_amdgcn_s_waitcnt(L::kWait);
        const PathInfo cur = pnext;
        const int clen = plen;
        lds_barrier();
        const int my_par = lane < N ? reinterpret_cast<const int*>(ldsb + L::kSM)[lane] : -1;
        const float my_alpha = lane < N ? reinterpret_cast<const float*>(ldsb + L::kSM + 256)[lane] : 1.0f;
        const float bl = lane < N ? reinterpret_cast<const float*>(ldsb + L::kSM + 512)[lane] : 0.0f;

        // ---- the sequence's tree (lane = node), once per run of its heads (the first run's
        // in the prologue)
        if (b != seq) {
            seq = b;
            head_tree<NKT>(my_par, N, lane, status, tr);
        }

        // ---- this head's gates: g_t = product of alpha over t's ancestors-or-self
        float g_l = lane < N ? my_alpha : 1.0f;
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            if (r < tr.grounds) {
                const int j = tr.jp[r];
                const float gj = __shfl(g_l, j < 0 ? lane : j);
                if (j >= 0) g_l *= gj;
            }
        }
        if (wave == 0 && lane < N) {
            gamma[(node0 + lane) * H + h] = g_l;
            if (h == 0) {
                if (anc_out) anc_out[node0 + lane] = tr.anc_l;
                if (depth_out) depth_out[node0 + lane] = __popcll(tr.anc_l);
            }
        }

        // ---- the previous step's commit on this head's rows
        if constexpr (FUSED && DEFER) {
            if (cur.depth + clen > 0) {
                head_commit_defer<NKT>(lds, cur, clen, cin, dlog, bh, H, wave, lane, lds_addr);
            } else if (wave == 0 && lane == 0) {    // nothing logged or accepted: S stays
                dlog.scale_out[bh] = reinterpret_cast<const float*>(ldsb + L::kLS)[0];
                if (h == 0) dlog.len_out[b] = 0;
            }
        } else if constexpr (FUSED) {
            if (cur.depth > 0) head_commit_rows<NKT>(lds, cur, cin, bh, H, wave, lane, lds_addr);
        }

        // ---- MFMA operands of this wave's 16 rows (committed, with FUSED)
        bf16x8_t ahi[4], alo[4];
        {
            const int r = 16 * wave + col;
            const float* rowp = lds + r * D;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int c0 = 2 * grp + 8 * ks;
                split_hi_lo(*reinterpret_cast<const f32x4_t*>(rowp + 4 * (c0 ^ (r & 15))),
                            *reinterpret_cast<const f32x4_t*>(rowp + 4 * ((c0 + 1) ^ (r & 15))),
                            ahi[ks], alo[ks]);
            }
        }
        lds_barrier();                        // S rows and path rows read: both may be refilled

        // ---- the next head's S rows (the first quarter) and path rows
        if (more) {
            issue_s_pairs<FUSED>(S0, lds_addr, bh + 1, 0, 0, kSParts == 4 ? 1 : 2, wave, lane);
            if constexpr (FUSED) {
                if ((bh + 1) / H != b) {
                    const int pidx = lane < cin.Np ? reinterpret_cast<const int*>(ldsb + L::kPI)[lane] : -1;
                    const int pacc = reinterpret_cast<const int*>(ldsb + L::kPA)[0];
                    pnext = fused_path(pidx, pacc, cin.Np, lane, wave == 0 && (bh + 1) % H == 0,
                                       status);
                    if constexpr (DEFER)
                        plen = head_log_len<NKT>(ldsb, dlog.Lmax,
                                                 wave == 0 && lane == 0 && (bh + 1) % H == 0, status);
                }
                if constexpr (DEFER)
                    head_issue_terms<NKT>(cin, dlog, pnext, plen, 0, bh + 1, H, wave, lane, lds_addr);
                else if (pnext.depth > 0)
                    head_issue_path<NKT>(cin, pnext, 0, bh + 1, H, wave, lane, lds_addr);
            }
        }

        // ---- the Gram tiles, scaled, into the coefficient tables.  They need the key/query
        // rows and the gates only, so they run after the next head's state rows are
        // requested: the transfer then has the whole rest of this head to arrive.  Key rows
        // 16 rt.. have NKT + 1 tiles (key-key at or left of the diagonal, key-query at or
        // right of it), dealt to the 8 / NKT waves of that row tile.
        {
            constexpr int kWavesPerRow = kHeadWaves / NKT;
            const int rtg = wave / kWavesPerRow;
            const int jg = wave - rtg * kWavesPerRow;
            if (16 * rtg < N && jg <= NKT) {
                uint64_t anc_me[4];
                float rgm[4], bgm[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = (16 * rtg + 4 * grp + e) & 63;
                    const uint64_t a = shfl_u64(tr.anc_l, m);
                    anc_me[e] = m < N ? a : 0ull;
                    const float gme = __shfl(g_l, m);
                    rgm[e] = __builtin_amdgcn_rcpf(gme);
                    bgm[e] = __shfl(bl, m) * gme;
                }
                bf16x8_t ka[4];
                {
                    const uint32_t m = 16u * rtg + col;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        ka[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                            ldsb + L::kKQ + 256 * m + 16 * ((4 * ks + grp) ^ (m & 15))));
                }
                for (int eg = jg; eg <= NKT; eg += kWavesPerRow) {
                    const bool is_q = eg > rtg;
                    const int ct = is_q ? eg - 1 : eg;
                    if (16 * ct >= N) continue;
                    const uint32_t n = 16u * ct + col;
                    const bool live = n < static_cast<uint32_t>(N);
                    const uint32_t r = (is_q ? static_cast<uint32_t>(NN) : 0u) + n;
                    bf16x8_t bv[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        bv[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                            ldsb + L::kKQ + 256 * r + 16 * ((4u * ks + grp) ^ (r & 15u))));
                    const uint64_t an0 = shfl_u64(tr.anc_l, static_cast<int>(n));
                    const float gn = __shfl(g_l, static_cast<int>(n));
                    const float rgn = __builtin_amdgcn_rcpf(gn);
                    f32x4_t gacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        gacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], bv[ks], gacc, 0, 0, 0);
                    const uint64_t an = live ? an0 : 0ull;      // node n = 16 ct + col
                    const int dn = __popcll(an);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = 16 * rtg + 4 * grp + e;   // key row
                        if (!is_q) {
                            // C[depth(n) - 1][t = m], n a strict ancestor of m
                            const bool need = live && m < N && ((anc_me[e] >> n) & 1ull) &&
                                              static_cast<int>(n) != m;
                            if (need && dn - 1 < kHeadSlots)
                                Ct[(dn - 1) * NN + m] = bgm[e] * rgn * gacc[e];
                        } else {
                            // W[depth(m) - 1][t = n], m an ancestor-or-self of n
                            const int dm = __popcll(anc_me[e]);
                            const bool need = live && m < N && ((an >> m) & 1ull);
                            if (need && dm - 1 < kHeadSlots)
                                Wt[(dm - 1) * NN + n] = gn * rgm[e] * gacc[e];
                        }
                    }
                }
            }
        }

        if constexpr (kSParts == 4) {
            if (more) issue_s_pairs<FUSED>(S0, lds_addr, bh + 1, 0, 2, 1, wave, lane);
        }

        // ---- contractions P = S K^T, Y = S Q^T on this wave's 16 rows (columns of nodes
        // past N come out of whatever those rows hold and are never used)
        f32x4_t acc[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            const uint32_t r = 16u * c + col;           // key rows, then query rows
            bf16x8_t bv[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                bv[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                    ldsb + L::kKQ + 256 * r + 16 * ((4u * ks + grp) ^ (r & 15u))));
            acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[ks], bv[ks], acc[c], 0, 0, 0);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[ks], bv[ks], acc[c], 0, 0, 0);
            }
        }
        if (more) issue_s_pairs<FUSED>(S0, lds_addr, bh + 1, 0, 4, kSParts == 4 ? 1 : 2, wave, lane);
        // this head's values: v of node 16 kt + col, rows 16 w + 4 grp .. +3
        uint2 vraw[NKT];
        {
            const uint32_t ch = 2u * wave + (static_cast<uint32_t>(grp) >> 1);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const uint32_t t = 16u * kt + col;
                vraw[kt] = *reinterpret_cast<const uint2*>(
                    ldsb + L::kV + 256u * t + 16u * (ch ^ (t & 15u)) + 8u * (grp & 1));
            }
        }
        lds_barrier();                        // coefficients visible; key/query/value rows,
                                              // parents and gates read

        // ---- the next head's last S-row quarter, key/query/value rows, parents and gates
        // (and, fused, the previous tree of the head after it)
        if (more) {
            if constexpr (kSParts == 4) issue_s_pairs<FUSED>(S0, lds_addr, bh + 1, 0, 6, 1, wave, lane);
            head_issue_inputs<NKT>(Q, K, V, alpha, beta, parent, H, N, bh + 1, wave, lane, lds_addr);
            if constexpr (FUSED) {
                if (bh + 2 < hi && wave == kHeadWaves - 1)
                    head_issue_prev_tree<NKT>(cin, bh + 2, H, lane, lds_addr, len_in);
            }
        }

        // ---- per lane: nodes t = 16 kt + col, rows v0..v0+3: right-hand sides and g_t Y
        float g_kt[NKT], b_kt[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            const int t = 16 * kt + col;
            g_kt[kt] = __shfl(g_l, t);
            b_kt[kt] = __shfl(bl, t);
        }
        float Uv[NKT][4], Ov[NKT][4];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            const int t = 16 * kt + col;
            const float vv[4] = {__uint_as_float(vraw[kt].x << 16), __uint_as_float(vraw[kt].x & 0xffff0000u),
                                 __uint_as_float(vraw[kt].y << 16), __uint_as_float(vraw[kt].y & 0xffff0000u)};
            const float bgt = b_kt[kt] * g_kt[kt];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Uv[kt][e] = b_kt[kt] * vv[e] - bgt * acc[kt][e];
                Ov[kt][e] = g_kt[kt] * acc[NKT + kt][e];
            }
            if (tr.dtk[kt] == 1)                  // a node of depth 1: its U is final already
                *reinterpret_cast<f32x4_t*>(Us + t * 16 + 4 * grp) =
                    f32x4_t{Uv[kt][0], Uv[kt][1], Uv[kt][2], Uv[kt][3]};
        }
        // ---- ancestor walk: step d folds in every node's depth-d ancestor (final since step
        // d - 1).  Up to depth kHeadList the ancestor comes from the node's packed list and
        // the coefficients from the tables; a node's U goes to the exchange once, when it is
        // final.  Lanes without an ancestor at this depth read node 0 (depth 1, always
        // written) with zero coefficients.
        int d = 1;
#pragma unroll
        for (int wd = 0; wd < kHeadListWords; ++wd) {
#pragma unroll
            for (int j = 0; j < kHeadListPer; ++j) {
                if (d < tr.maxd) {
                    float cs[NKT], cw[NKT];
                    f32x4_t x[NKT];
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt) {
                        const int t = 16 * kt + col;
                        const int a = static_cast<int>((tr.alist[kt][wd] >> (6 * j)) & 63u);
                        const bool has = d < tr.dtk[kt];
                        x[kt] = *reinterpret_cast<const f32x4_t*>(Us + a * 16 + 4 * grp);
                        const float c = Ct[(d - 1) * NN + t];
                        const float w = Wt[(d - 1) * NN + t];
                        cs[kt] = has ? c : 0.f;
                        cw[kt] = has ? w : 0.f;
                    }
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            Uv[kt][e] -= cs[kt] * x[kt][e];
                            Ov[kt][e] += cw[kt] * x[kt][e];
                        }
                        if (d + 1 == tr.dtk[kt])  // that was its last ancestor: U is final
                            *reinterpret_cast<f32x4_t*>(Us + (16 * kt + col) * 16 + 4 * grp) =
                                f32x4_t{Uv[kt][0], Uv[kt][1], Uv[kt][2], Uv[kt][3]};
                    }
                    ++d;
                }
            }
        }
        // deeper trees: the depth-d ancestor from the mask, the coefficients from the key and
        // query rows in memory
        const uint16_t* Kh = K + (node0 * H + h) * D;
        const uint16_t* Qh = Q + (node0 * H + h) * D;
        const size_t nstride = static_cast<size_t>(H) * D;
        for (; d < tr.maxd; ++d) {
            float cs[NKT], cw[NKT];
            f32x4_t x[NKT];
            bool fin[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const int tn = 16 * kt + col;
                const uint64_t at = shfl_u64(tr.anc_l, tn);
                uint64_t m = tn < N ? (at & ~(1ull << tn)) : 0ull;
                for (int i = 1; i < d; ++i) m &= m - 1ull;       // drop the shallower ancestors
                const bool has = m != 0ull;
                fin[kt] = has && (m & (m - 1ull)) == 0ull;
                // lanes without an ancestor here read node 0's rows (nothing past N)
                const int t = has ? tn : 0;
                const int a = has ? __ffsll(static_cast<unsigned long long>(m)) - 1 : 0;
                const float rga = __builtin_amdgcn_rcpf(__shfl(g_l, a));
                const float kk = head_dot_bf16(Kh + t * nstride, Kh + a * nstride, grp);
                const float kq = head_dot_bf16(Kh + a * nstride, Qh + t * nstride, grp);
                cs[kt] = has ? b_kt[kt] * g_kt[kt] * rga * kk : 0.f;
                cw[kt] = has ? g_kt[kt] * rga * kq : 0.f;
                x[kt] = *reinterpret_cast<const f32x4_t*>(Us + a * 16 + 4 * grp);
            }
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Uv[kt][e] -= cs[kt] * x[kt][e];
                    Ov[kt][e] += cw[kt] * x[kt][e];
                }
                if (fin[kt])
                    *reinterpret_cast<f32x4_t*>(Us + (16 * kt + col) * 16 + 4 * grp) =
                        f32x4_t{Uv[kt][0], Uv[kt][1], Uv[kt][2], Uv[kt][3]};
            }
        }
        // ---- the node's own term; then O and U out as whole rows.  A wave holds 16 values
        // of each node, so its own stores would cover only 64 of a row's 512 bytes; the rows
        // are assembled in the U exchange instead and each wave writes eight whole rows,
        // with the streaming hint (written once, not read again by this launch)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            const int t = 16 * kt + col;
            const bool ok = t < N;
            const int dt = tr.dtk[kt];
            const bool in_table = ok && dt - 1 < kHeadSlots;
            float cw = in_table ? Wt[(dt - 1) * NN + t] : 0.f;
            if (tr.maxd > kHeadSlots) {           // (uniform) the node's own k.q from memory
                const int tt = ok ? t : 0;
                const float kq = head_dot_bf16(Kh + tt * nstride, Qh + tt * nstride, grp);
                if (ok && !in_table) cw = kq;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Ov[kt][e] += cw * Uv[kt][e];
        }
        const size_t row0 = (node0 * H + h) * D;
        if constexpr (L::kOwnO) {
            float* Os = reinterpret_cast<float*>(ldsb + L::kO) + wave * (NN * 16);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                *reinterpret_cast<f32x4_t*>(Os + (16 * kt + col) * 16 + 4 * grp) =
                    f32x4_t{Ov[kt][0], Ov[kt][1], Ov[kt][2], Ov[kt][3]};
            lds_barrier();                    // every wave's U and O rows in their exchanges
            head_store_rows<NKT>(U + row0, ldsb, H, N, wave, lane);
            head_store_rows<NKT>(O + row0, ldsb, H, N, wave, lane, L::kO);
        } else {
            lds_barrier();                    // every wave's U rows are in its exchange area
            head_store_rows<NKT>(U + row0, ldsb, H, N, wave, lane);
            lds_barrier();                    // ... and have been read
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                *reinterpret_cast<f32x4_t*>(Us + (16 * kt + col) * 16 + 4 * grp) =
                    f32x4_t{Ov[kt][0], Ov[kt][1], Ov[kt][2], Ov[kt][3]};
            lds_barrier();                    // O rows in the exchange
            head_store_rows<NKT>(O + row0, ldsb, H, N, wave, lane);
        }
        if (!more) break;
        ++bh;
    }
}

// Compute units of the current device, queried once per device.  The cache entries are
// atomics: concurrent first calls from several host threads may each query the attribute,
// and all store the same value.
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

template <int NCT, int MODE, int NFIX = 0>
static hipError_t launch_small(const VerifyArgs& a, const CommitIn& cin, const DeferLog& dl,
                               hipStream_t stream) {
    const SmallLds L = small_lds(a.N, NCT, MODE, MODE == 2 ? dl.Lmax : 0);
    const int bytes = static_cast<int>(L.bytes);
    const int wgs = small_wgs(L.bytes, kSmallWavesPerSimd<NCT, MODE>);
    auto kern = verify_small_kernel<NCT, MODE, NFIX>;
    if (L.bytes > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) return e;
    }
    const int BH = a.B * a.H;
    const int items = BH * kSmallParts;
    const int slots = wgs * device_cu_count();   // resident workgroups
    const int grid = items < slots ? items : slots;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kSmallThreads), bytes, stream, a.S0,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), a.alpha, a.beta, a.parent, a.H, a.N,
                       BH, a.O, a.U, a.gamma, a.anc_out, a.depth_out, a.status, cin, dl);
    return hipGetLastError();
}


// Trees of up to 8 nodes: the small-tree kernel compiled for the exact node count.
template <int MODE>
static hipError_t launch_small_fixed(const VerifyArgs& a, const CommitIn& cin, const DeferLog& dl,
                                     hipStream_t stream) {
    switch (a.N) {
        case 1: return launch_small<1, MODE, 1>(a, cin, dl, stream);
        case 2: return launch_small<1, MODE, 2>(a, cin, dl, stream);
        case 3: return launch_small<1, MODE, 3>(a, cin, dl, stream);
        case 4: return launch_small<1, MODE, 4>(a, cin, dl, stream);
        case 5: return launch_small<1, MODE, 5>(a, cin, dl, stream);
        case 6: return launch_small<1, MODE, 6>(a, cin, dl, stream);
        case 7: return launch_small<1, MODE, 7>(a, cin, dl, stream);
        default: return launch_small<1, MODE, 8>(a, cin, dl, stream);
    }
}

}  // namespace

template <bool FUSED>
static hipError_t launch_f32(const VerifyArgs& a, const CommitInF32& cin, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H) * kF32Blocks;
    if (a.N <= kTinyN && (!FUSED || cin.Np <= kTinyN)) {
        hipLaunchKernelGGL(verify_f32_tiny_kernel<FUSED>, dim3(grid), dim3(kF32Threads), 0, stream,
                           a.S0, static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                           static_cast<const float*>(a.V), a.alpha, a.beta, a.parent, a.H, a.N,
                           a.O, a.U, a.gamma, a.anc_out, a.depth_out, a.status, cin);
        return hipGetLastError();
    }
    const F32Lds L = f32_lds(a.N);
    auto kern = verify_f32_kernel<FUSED>;
    if (L.bytes > 48u * 1024u) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(L.bytes));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kF32Threads), L.bytes, stream, a.S0,
                       static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                       static_cast<const float*>(a.V), a.alpha, a.beta, a.parent, a.H, a.N, a.O,
                       a.U, a.gamma, a.anc_out, a.depth_out, a.status, cin);
    return hipGetLastError();
}

template <int NKT>
static hipError_t launch_large(const VerifyArgs& a, hipStream_t stream) {
    const size_t dyn = sizeof(float) * LargeLayout<NKT>::kTotal;
    auto kern = verify_large_kernel<NKT>;
    const int BH = a.B * a.H;
    const int items = BH * kSmallParts;
    // resident workgroups per CU: three (registers), within the 160 KB of LDS
    const int slots = small_wgs(dyn, 3) * device_cu_count();
    const int grid = items < slots ? items : slots;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kSmallThreads), dyn, stream, a.S0,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), a.alpha, a.beta, a.parent, a.H, a.N,
                       BH, a.O, a.U, a.gamma, a.anc_out, a.depth_out, a.status);
    return hipGetLastError();
}

template <int NKT, bool FUSED, bool DEFER = false>
static hipError_t launch_head(const VerifyArgs& a, hipStream_t stream, const CommitIn* cin = nullptr,
                              const DeferLog* dl = nullptr) {
    using L = HeadLds<NKT>;
    auto kern = verify_head_kernel<NKT, FUSED, DEFER>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(L::kBytes));
    if (e != hipSuccess) return e;
    const int BH = a.B * a.H;
    const int cus = device_cu_count();          // one workgroup per CU (LDS)
    const int grid = BH < cus ? BH : cus;
    // the fused commit of a path of up to eight nodes: on the vector ALUs (less latency)
    // unless each workgroup has at least 32 heads, where the matrix-core form measured faster
    // (B256 x H64 32-node trees 604 -> 599 us; B128 x H32 64-node trees 217 -> 219 us and
    // B32 x H32 21-node trees 41.4 -> 43.5 us the other way)
    CommitIn c = cin ? *cin : CommitIn{};
    c.short_path = BH < 32 * cus ? 8 : 0;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kHeadThreads), L::kBytes, stream, a.S0,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), a.alpha, a.beta, a.parent, a.H, a.N,
                       BH, a.O, a.U, a.gamma, a.anc_out, a.depth_out, a.status,
                       c, dl ? *dl : DeferLog{});
    return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    if (a.in_dtype != TREEWY_BF16) return launch_f32<false>(a, CommitInF32{}, stream);
    const CommitIn none{};
    const DeferLog nolog{};
    if (a.N <= 8) return launch_small_fixed<0>(a, none, nolog, stream);
    if (a.N <= 16) return launch_small<2, 0>(a, none, nolog, stream);
    // 17-32 nodes: items of half a head, three workgroups per CU (the key and query rows go
    // through the S-row area, no LDS area of their own); this measured faster for the plain
    // verify than one head per item.  33-48 and 49-64 nodes: one head per item, three or
    // four node tiles.
    if (a.N <= 32) return launch_large<2>(a, stream);
    if (a.N <= 48) return launch_head<3, false>(a, stream);
    return launch_head<4, false>(a, stream);
}

// The previous step's commit fused into this step's verify: one kernel for every tree size
// and input type.
hipError_t launch_commit_verify(const CommitArgs& c, const VerifyArgs& a, hipStream_t stream) {
    if (a.in_dtype == TREEWY_BF16 && a.N <= 16) {
        const CommitIn cin{c.S, c.U, static_cast<const uint16_t*>(c.K), c.gamma, c.parent,
                           c.accepted, c.N};
        const DeferLog nolog{};
        if (a.N <= 8) return launch_small_fixed<1>(a, cin, nolog, stream);
        return launch_small<2, 1>(a, cin, nolog, stream);
    }
    if (a.in_dtype == TREEWY_BF16) {
        const CommitIn cin{c.S, c.U, static_cast<const uint16_t*>(c.K), c.gamma, c.parent,
                           c.accepted, c.N};
        // 17-64 nodes: one head per item (at 17-32 nodes this measured faster than items of
        // half a head for the fused step, B256 x H64 32-node trees 637 -> 604 us, while the
        // plain verify above keeps the half-head items)
        if (a.N <= 32) return launch_head<2, true>(a, stream, &cin);
        if (a.N <= 48) return launch_head<3, true>(a, stream, &cin);
        return launch_head<4, true>(a, stream, &cin);
    }
    const CommitInF32 cin{c.S, c.U, static_cast<const float*>(c.K), c.gamma, c.parent,
                          c.accepted, c.N};
    return launch_f32<true>(a, cin, stream);
}

// The deferred commit (bf16 inputs: the caller checks), on the kernel of the fused path for
// the tree size.
hipError_t launch_commit_verify_deferred(const CommitArgs& c, const VerifyArgs& a,
                                         const DeferArgs& d, hipStream_t stream) {
    const CommitIn cin{c.S, c.U, static_cast<const uint16_t*>(c.K), c.gamma, c.parent,
                       c.accepted, c.N};
    const DeferLog dl{d.logU, static_cast<uint16_t*>(d.logK), d.scale_in, d.scale_out,
                      d.len_in, d.len_out, d.Lmax};
    if (a.N <= 8) return launch_small_fixed<2>(a, cin, dl, stream);
    if (a.N <= 16) return launch_small<2, 2>(a, cin, dl, stream);
    if (a.N <= 32) return launch_head<2, true, true>(a, stream, &cin, &dl);
    if (a.N <= 48) return launch_head<3, true, true>(a, stream, &cin, &dl);
    return launch_head<4, true, true>(a, stream, &cin, &dl);
}

}  // namespace treewy
