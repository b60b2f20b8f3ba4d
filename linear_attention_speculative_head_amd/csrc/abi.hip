// C ABI of the TreeWY path (declared in include/treewy.h): host-side argument checks,
// then one kernel launch on the caller's stream.  No allocation, no synchronisation, no
// host read of device memory.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "treewy.h"

namespace {

// A launch covers up to 2*B*H workgroups of 256 lanes; the dispatch grid is counted in
// lanes and must fit 32 bits.
bool sizes_ok(int B, int H, int N) {
    // H <= 65536 keeps a node's byte offset within one sequence's rows (node x H x 512 B for
    // fp32 rows) inside the 32-bit offsets of the kernels' transfers and range-checked stores
    if (B < 1 || H < 1 || H > 65536 || N < 1 || N > 64) return false;
    const uint64_t groups = static_cast<uint64_t>(B) * static_cast<uint64_t>(H);
    return groups * 2u * 256u <= 0xffffffffull;
}

bool dtype_ok(int d) { return d == TREEWY_F32 || d == TREEWY_BF16; }

int map_hip(hipError_t e) { return e == hipSuccess ? TREEWY_OK : TREEWY_EHIP; }

constexpr size_t D_ROW = 128;   // elements per node row

struct Span {
    const void* p;
    size_t bytes;
};

bool overlap(const Span& x, const Span& y) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), b0 = reinterpret_cast<uintptr_t>(y.p);
    return a0 < b0 + y.bytes && b0 < a0 + x.bytes;
}

}  // namespace

extern "C" {

int treewy_verify(const float* S0, const void* Q, const void* K, const void* V,
                  const float* alpha, const float* beta, const int32_t* parent, int B, int H,
                  int N, int in_dtype, float* O, float* U, float* gamma, uint64_t* anc_out,
                  int32_t* depth_out, int32_t* status, void* stream)
{
    if (!S0 || !Q || !K || !V || !alpha || !beta || !parent || !O || !U || !gamma)
        return TREEWY_EINVAL;
    if (!sizes_ok(B, H, N) || !dtype_ok(in_dtype)) return TREEWY_EINVAL;
    treewy::VerifyArgs a{S0, Q, K, V, alpha, beta, parent, B, H, N, in_dtype,
                         O, U, gamma, anc_out, depth_out, status};
    return map_hip(treewy::launch_verify(a, static_cast<hipStream_t>(stream)));
}

int treewy_commit(float* S, const float* U, const void* K, const float* gamma,
                  const int32_t* parent, const int32_t* accepted, int B, int H, int N,
                  int in_dtype, int32_t* status, void* stream)
{
    if (!S || !U || !K || !gamma || !parent || !accepted) return TREEWY_EINVAL;
    if (!sizes_ok(B, H, N) || !dtype_ok(in_dtype)) return TREEWY_EINVAL;
    treewy::CommitArgs a{S, U, K, gamma, parent, accepted, B, H, N, in_dtype, status};
    return map_hip(treewy::launch_commit(a, static_cast<hipStream_t>(stream)));
}

int treewy_commit_verify(float* S, const float* U_prev, const void* K_prev,
                         const float* gamma_prev, const int32_t* parent_prev,
                         const int32_t* accepted_prev, int N_prev, const void* Q, const void* K,
                         const void* V, const float* alpha, const float* beta,
                         const int32_t* parent, int B, int H, int N, int in_dtype, float* O,
                         float* U, float* gamma, uint64_t* anc_out, int32_t* depth_out,
                         int32_t* status, void* stream)
{
    if (!S || !U_prev || !K_prev || !gamma_prev || !parent_prev || !accepted_prev || !Q || !K ||
        !V || !alpha || !beta || !parent || !O || !U || !gamma)
        return TREEWY_EINVAL;
    if (!sizes_ok(B, H, N) || !sizes_ok(B, H, N_prev) || !dtype_ok(in_dtype)) return TREEWY_EINVAL;
    // this step's outputs must not overwrite the previous step's factors while they are read
    const size_t esz = in_dtype == TREEWY_BF16 ? 2 : 4;
    const size_t rows = static_cast<size_t>(B) * H * D_ROW;
    const Span outs[3] = {{O, rows * N * 4}, {U, rows * N * 4},
                          {gamma, static_cast<size_t>(B) * N * H * 4}};
    const Span ins[3] = {{U_prev, rows * N_prev * 4}, {K_prev, rows * N_prev * esz},
                         {gamma_prev, static_cast<size_t>(B) * N_prev * H * 4}};
    for (const Span& o : outs)
        for (const Span& i : ins)
            if (overlap(o, i)) return TREEWY_EINVAL;
    treewy::CommitArgs c{S, U_prev, K_prev, gamma_prev, parent_prev, accepted_prev, B, H, N_prev,
                         in_dtype, status};
    treewy::VerifyArgs a{S, Q, K, V, alpha, beta, parent, B, H, N, in_dtype,
                         O, U, gamma, anc_out, depth_out, status};
    return map_hip(treewy::launch_commit_verify(c, a, static_cast<hipStream_t>(stream)));
}

int treewy_commit_verify_deferred(float* S, float* logU, void* logK, const float* scale_in,
                                  float* scale_out, const int32_t* len_in, int32_t* len_out,
                                  int Lmax, const float* U_prev, const void* K_prev,
                                  const float* gamma_prev, const int32_t* parent_prev,
                                  const int32_t* accepted_prev, int N_prev, const void* Q,
                                  const void* K, const void* V, const float* alpha,
                                  const float* beta, const int32_t* parent, int B, int H, int N,
                                  int in_dtype, float* O, float* U, float* gamma,
                                  uint64_t* anc_out, int32_t* depth_out, int32_t* status,
                                  void* stream)
{
    if (!S || !logU || !logK || !scale_in || !scale_out || !len_in || !len_out || !U_prev ||
        !K_prev || !gamma_prev || !parent_prev || !accepted_prev || !Q || !K || !V || !alpha ||
        !beta || !parent || !O || !U || !gamma)
        return TREEWY_EINVAL;
    if (!sizes_ok(B, H, N) || !sizes_ok(B, H, N_prev) || in_dtype != TREEWY_BF16 ||
        Lmax < 1 || Lmax > 16)
        return TREEWY_EINVAL;
    const size_t rows = static_cast<size_t>(B) * H * D_ROW;
    const size_t heads = static_cast<size_t>(B) * H;
    // this step's outputs must not overwrite the previous step's factors while they are read,
    // and the header is read from one buffer and written to another
    const Span outs[5] = {{O, rows * N * 4}, {U, rows * N * 4},
                          {gamma, static_cast<size_t>(B) * N * H * 4},
                          {scale_out, heads * 4}, {len_out, static_cast<size_t>(B) * 4}};
    const Span ins[5] = {{U_prev, rows * N_prev * 4}, {K_prev, rows * N_prev * 2},
                         {gamma_prev, static_cast<size_t>(B) * N_prev * H * 4},
                         {scale_in, heads * 4}, {len_in, static_cast<size_t>(B) * 4}};
    for (const Span& o : outs)
        for (const Span& i : ins)
            if (overlap(o, i)) return TREEWY_EINVAL;
    treewy::CommitArgs c{S, U_prev, K_prev, gamma_prev, parent_prev, accepted_prev, B, H, N_prev,
                         in_dtype, status};
    treewy::VerifyArgs a{S, Q, K, V, alpha, beta, parent, B, H, N, in_dtype,
                         O, U, gamma, anc_out, depth_out, status};
    treewy::DeferArgs d{logU, logK, scale_in, scale_out, len_in, len_out, Lmax};
    return map_hip(treewy::launch_commit_verify_deferred(c, a, d, static_cast<hipStream_t>(stream)));
}

int treewy_deferred_flush(float* S, const float* logU, const void* logK, const float* scale_in,
                          float* scale_out, const int32_t* len_in, int32_t* len_out, int Lmax,
                          int B, int H, int in_dtype, int32_t* status, void* stream)
{
    if (!S || !logU || !logK || !scale_in || !scale_out || !len_in || !len_out) return TREEWY_EINVAL;
    if (!sizes_ok(B, H, 1) || in_dtype != TREEWY_BF16 || Lmax < 1 || Lmax > 16) return TREEWY_EINVAL;
    const size_t heads = static_cast<size_t>(B) * H;
    if (overlap({scale_out, heads * 4}, {scale_in, heads * 4}) ||
        overlap({len_out, static_cast<size_t>(B) * 4}, {len_in, static_cast<size_t>(B) * 4}) ||
        overlap({scale_out, heads * 4}, {len_in, static_cast<size_t>(B) * 4}) ||
        overlap({len_out, static_cast<size_t>(B) * 4}, {scale_in, heads * 4}))
        return TREEWY_EINVAL;
    treewy::DeferArgs d{const_cast<float*>(logU), const_cast<void*>(logK), scale_in, scale_out,
                        len_in, len_out, Lmax};
    return map_hip(treewy::launch_deferred_flush(S, d, B, H, in_dtype, status,
                                                 static_cast<hipStream_t>(stream)));
}

int treewy_verify_snapshot(const float* S0, const void* Q, const void* K, const void* V,
                           const float* alpha, const float* beta, const int32_t* parent,
                           int B, int H, int N, int in_dtype, float* O, float* Snap,
                           int32_t* status, void* stream)
{
    if (!S0 || !Q || !K || !V || !alpha || !beta || !parent || !O || !Snap) return TREEWY_EINVAL;
    if (!sizes_ok(B, H, N) || !dtype_ok(in_dtype)) return TREEWY_EINVAL;
    treewy::SnapshotVerifyArgs a{S0, Q, K, V, alpha, beta, parent, B, H, N, in_dtype,
                                 O, Snap, status};
    return map_hip(treewy::launch_verify_snapshot(a, static_cast<hipStream_t>(stream)));
}

int treewy_commit_snapshot(float* S, const float* Snap, const int32_t* accepted, int B, int H,
                           int N, int32_t* status, void* stream)
{
    if (!S || !Snap || !accepted) return TREEWY_EINVAL;
    if (!sizes_ok(B, H, N)) return TREEWY_EINVAL;
    treewy::SnapshotCommitArgs a{S, Snap, accepted, B, H, N, status};
    return map_hip(treewy::launch_commit_snapshot(a, static_cast<hipStream_t>(stream)));
}

size_t treewy_tree_attention_workspace(int B, int Hkv, int G, int N, int T_max)
{
    if (B < 1 || Hkv < 1 || G < 1 || N < 1 || N > 64 || T_max < 1) return 0;
    return treewy::attention_workspace_bytes(B, Hkv, G, N, T_max);
}

namespace {

bool attn_sizes_ok(int B, int Hkv, int G, int N, int T_max) {
    if (B < 1 || Hkv < 1 || G < 1 || N < 1 || N > 64 || T_max < 1) return false;
    const uint64_t bk = static_cast<uint64_t>(B) * Hkv;
    const uint64_t nq = static_cast<uint64_t>(N) * G;
    // grid limits (query blocks and B*Hkv in y/z) and 32-bit element offsets per head row
    return bk <= 65535u && (nq + 31) / 32 <= 65535u &&
           static_cast<uint64_t>(T_max) * 256u * 2u <= 0x7fffffffull;
}

}  // namespace

int treewy_tree_attention(const void* Kc, const void* Vc, const int32_t* ctx, int T_max,
                          const void* Qd, const void* Kd, const void* Vd, const int32_t* parent,
                          int B, int Hkv, int G, int N, float* O, void* workspace,
                          size_t workspace_bytes, int32_t* status, void* stream)
{
    if (!Kc || !Vc || !ctx || !Qd || !Kd || !Vd || !parent || !O || !workspace) return TREEWY_EINVAL;
    if (!attn_sizes_ok(B, Hkv, G, N, T_max)) return TREEWY_EINVAL;
    if (workspace_bytes < treewy::attention_workspace_bytes(B, Hkv, G, N, T_max)) return TREEWY_EINVAL;
    treewy::AttentionArgs a{Kc, Vc, ctx, T_max, Qd, Kd, Vd, parent, B, Hkv, G, N, O, workspace,
                            status};
    return map_hip(treewy::launch_tree_attention(a, static_cast<hipStream_t>(stream)));
}

int treewy_tree_attention_noalloc(const void* Kc, const void* Vc, const int32_t* ctx, int T_max,
                                  const void* Qd, const void* Kd, const void* Vd,
                                  const int32_t* parent, int B, int Hkv, int G, int N, float* O,
                                  int32_t* status, void* stream)
{
    if (!Kc || !Vc || !ctx || !Qd || !Kd || !Vd || !parent || !O) return TREEWY_EINVAL;
    if (!attn_sizes_ok(B, Hkv, G, N, T_max)) return TREEWY_EINVAL;
    if (treewy::attention_workspace_bytes(B, Hkv, G, N, T_max) > TREEWY_NOALLOC_SCRATCH_BYTES)
        return TREEWY_ESCRATCH;
    treewy::AttentionArgs a{Kc, Vc, ctx, T_max, Qd, Kd, Vd, parent, B, Hkv, G, N, O, nullptr,
                            status};
    return map_hip(treewy::launch_tree_attention_noalloc(a, static_cast<hipStream_t>(stream)));
}

int treewy_kv_commit(void* Kc, void* Vc, const int32_t* ctx_in, int32_t* ctx_out, int T_max,
                     const void* Kd, const void* Vd, const int32_t* parent,
                     const int32_t* accepted, int B, int Hkv, int N, int32_t* status, void* stream)
{
    if (!Kc || !Vc || !ctx_in || !ctx_out || !Kd || !Vd || !parent || !accepted) return TREEWY_EINVAL;
    if (!attn_sizes_ok(B, Hkv, 1, N, T_max)) return TREEWY_EINVAL;
    if (overlap({ctx_in, static_cast<size_t>(B) * 4}, {ctx_out, static_cast<size_t>(B) * 4}))
        return TREEWY_EINVAL;
    treewy::KvCommitArgs a{Kc, Vc, ctx_in, ctx_out, T_max, Kd, Vd, parent, accepted, B, Hkv, N,
                           status};
    return map_hip(treewy::launch_kv_commit(a, static_cast<hipStream_t>(stream)));
}

const char* treewy_strerror(int code)
{
    switch (code) {
        case TREEWY_OK: return "success";
        case TREEWY_EINVAL: return "invalid argument (null pointer, size or dtype)";
        case TREEWY_EHIP: return "HIP launch or runtime error";
        case TREEWY_ETREE: return "malformed draft tree (parent outside [-1, t-1])";
        case TREEWY_EACCEPT: return "accepted node outside [-1, N-1]";
        case TREEWY_ELOG: return "deferred-commit log length outside [0, Lmax]";
        case TREEWY_ECTX: return "committed cache length outside [0, T_max] (or a path that does not fit)";
        case TREEWY_ESCRATCH: return "sizes need more split partials than the fixed device array of treewy_tree_attention_noalloc holds";
        default: return "unknown error code";
    }
}

int treewy_version(void) { return TREEWY_VERSION; }

}  // extern "C"
