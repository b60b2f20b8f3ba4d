// Internal launch interface between the C ABI (abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treewy.h"

namespace treewy {

struct VerifyArgs {
    const float* S0;
    const void* Q;
    const void* K;
    const void* V;
    const float* alpha;
    const float* beta;
    const int32_t* parent;
    int B, H, N, in_dtype;
    float* O;
    float* U;
    float* gamma;
    uint64_t* anc_out;
    int32_t* depth_out;
    int32_t* status;
};

struct CommitArgs {
    float* S;
    const float* U;
    const void* K;
    const float* gamma;
    const int32_t* parent;
    const int32_t* accepted;
    int B, H, N, in_dtype;
    int32_t* status;
};

struct SnapshotVerifyArgs {
    const float* S0;
    const void* Q;
    const void* K;
    const void* V;
    const float* alpha;
    const float* beta;
    const int32_t* parent;
    int B, H, N, in_dtype;
    float* O;
    float* Snap;
    int32_t* status;
};

struct SnapshotCommitArgs {
    float* S;
    const float* Snap;
    const int32_t* accepted;
    int B, H, N;
    int32_t* status;
};

// the log of the deferred commit (treewy_commit_verify_deferred)
struct DeferArgs {
    float* logU;
    void* logK;
    const float* scale_in;
    float* scale_out;
    const int32_t* len_in;
    int32_t* len_out;
    int Lmax;
};

// the tree-aware softmax-attention verify and its cache commit
struct AttentionArgs {
    const void* Kc;
    const void* Vc;
    const int32_t* ctx;
    int T_max;
    const void* Qd;
    const void* Kd;
    const void* Vd;
    const int32_t* parent;
    int B, Hkv, G, N;
    float* O;
    void* work;
    int32_t* status;
};

struct KvCommitArgs {
    void* Kc;
    void* Vc;
    const int32_t* ctx_in;
    int32_t* ctx_out;
    int T_max;
    const void* Kd;
    const void* Vd;
    const int32_t* parent;
    const int32_t* accepted;
    int B, Hkv, N;
    int32_t* status;
};

size_t attention_workspace_bytes(int B, int Hkv, int G, int N, int T_max);
hipError_t launch_tree_attention(const AttentionArgs& a, hipStream_t stream);
// the same with the partials in the library's fixed device array (a.work is ignored; the
// caller checks that attention_workspace_bytes fits kNoallocScratchBytes)
constexpr size_t kNoallocScratchBytes = TREEWY_NOALLOC_SCRATCH_BYTES;
hipError_t launch_tree_attention_noalloc(const AttentionArgs& a, hipStream_t stream);
hipError_t launch_kv_commit(const KvCommitArgs& a, hipStream_t stream);

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_commit(const CommitArgs& a, hipStream_t stream);
hipError_t launch_verify_snapshot(const SnapshotVerifyArgs& a, hipStream_t stream);
hipError_t launch_commit_snapshot(const SnapshotCommitArgs& a, hipStream_t stream);
// the commit described by `c` (its S, U, K, gamma, parent, accepted and node count N of the
// previous step), then the verify described by `a` on the committed state (a.S0 == c.S)
hipError_t launch_commit_verify(const CommitArgs& c, const VerifyArgs& a, hipStream_t stream);
// the same with the commit deferred into the log `d` (bf16 inputs, N <= 16)
hipError_t launch_commit_verify_deferred(const CommitArgs& c, const VerifyArgs& a,
                                         const DeferArgs& d, hipStream_t stream);
// the state the log stands for, written into S; the log is emptied into d's output header
hipError_t launch_deferred_flush(float* S, const DeferArgs& d, int B, int H, int in_dtype,
                                 int32_t* status, hipStream_t stream);

}  // namespace treewy
