// Internal interface between the C ABI layer (gdn_api.cpp) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

enum DType : int32_t { DT_FP32 = 0, DT_BF16 = 1, DT_FP16 = 2 };

constexpr int kChunk = 64;                  // chunk length C
constexpr int32_t kFlagQkL2Norm = 1;        // GDN_QK_L2NORM
constexpr int kTriTiles = 10;               // 16x16 tiles in the lower triangle of a C x C block
constexpr int kTileElems = 256;             // 16 x 16

struct DecodeArgs {
    int32_t N, H, dk, dv, in_dtype, out_dtype, flags;
    float *state;
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    void *o;
};

struct ChunkArgs {
    int32_t B, T, H, dk, dv, N, in_dtype, out_dtype, flags;
    const void *q, *k, *v;
    const float *log_alpha, *beta, *init_state;
    const int32_t *cu_seqlens;
    void *o;
    float *final_state;
    void *workspace;
};

// Workspace carve-up for one gdn_chunk_fwd call (byte offsets from the base).
struct ChunkWorkspace {
    int64_t max_rows;   // upper bound on (sequence, chunk) rows
    size_t off_meta, off_cu, off_row0, off_rowtok, off_rowlen, off_g, off_m, off_p, total;
};
ChunkWorkspace chunk_workspace_layout(int32_t B, int32_t T, int32_t N, bool packed, int32_t H,
                                      int32_t in_dtype);

hipError_t launch_decode_step(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t stream);
// Token-serial chunk call for batches of short sequences (meta: the
// workspace's status words; read when cu_seqlens is given, else written).
hipError_t launch_chunk_short(const ChunkArgs &a, int32_t *meta, hipStream_t stream);
// Average tokens per sequence up to which gdn_chunk_fwd runs token-serially.
constexpr int kShortAvg = 16;

// Host-side launch timing (see gdn_profile_* in gdn.h).  While profiling is
// enabled the scope records a HIP event pair around the launches it covers.
struct ProfScope {
    ProfScope(const char *name, hipStream_t stream);
    ~ProfScope();
    const char *name_;
    hipStream_t stream_;
    void *begin_;
};

}  // namespace gdn
