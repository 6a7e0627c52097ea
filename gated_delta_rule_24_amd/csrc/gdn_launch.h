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

// Token start and length of chunk row `row`.  With cpr > 0 the batch is
// B sequences of T tokens each, cpr = ceil(T / C) rows per sequence, and the
// span follows from the index; cpr = 0 reads the packed table.
__device__ __forceinline__ void row_span(int row, int T, int cpr, const int32_t *__restrict__ row_tok,
                                         const int32_t *__restrict__ row_len, int &tok0, int &len) {
    if (cpr) {
        const int s = row / cpr, c = row - s * cpr;
        tok0 = s * T + c * kChunk;
        len = min(kChunk, T - c * kChunk);
    } else {
        tok0 = row_tok[row];
        len = row_len[row];
    }
}

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
// With a segmented state pass (seg_chunks > 0) each sequence's chunks are cut
// into segments of seg_chunks chunks; a "segment unit" is one (sequence,
// segment) pair and max_units bounds their number (per head).
struct ChunkWorkspace {
    int64_t max_rows;    // upper bound on (sequence, chunk) rows
    int32_t seg_chunks;  // chunks per segment, 0 = one segment per sequence
    int64_t max_units;   // upper bound on segment units (0 when not segmented)
    size_t off_meta, off_cu, off_row0, off_rowtok, off_rowlen, off_g, off_m, off_p;
    size_t off_segfirst, off_segcnt, off_segtab;   // packed: first unit and unit count per sequence, unit -> (n, s)
    size_t off_end;      // per (unit, head): the segment's map [S-part; F-part], (dv + dk) x dk fp32
    size_t off_sin;      // per (unit, head): the state entering the segment, dv x dk fp32
    size_t total;
};
ChunkWorkspace chunk_workspace_layout(int32_t B, int32_t T, int32_t N, bool packed, int32_t H,
                                      int32_t in_dtype, int32_t dk, int32_t dv);
// Chunks per segment that gdn_chunk_fwd uses for this shape (0 = unsegmented).
int32_t chunk_seg_chunks(int32_t B, int32_t T, int32_t N, bool packed, int32_t H, int32_t dv);

hipError_t launch_decode_step(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t stream);
// Token-serial chunk call for batches of short sequences (meta: the
// workspace's status words; read when cu_seqlens is given, else written).
hipError_t launch_chunk_short(const ChunkArgs &a, int32_t *meta, hipStream_t stream);
// Average tokens per sequence up to which gdn_chunk_fwd runs token-serially.
constexpr int kShortAvg = 16;

// Backward pass (gdn_chunk_bwd): the incoming gradients and the gradients it writes.
struct BwdArgs {
    const float *d_o, *d_final;
    float *dq, *dk, *dv, *dlog_alpha, *dbeta, *d_init;
};

// Workspace carve-up for one gdn_chunk_bwd call: the chunk table of the
// forward layout, then per (chunk row, head) T, P, G and the decay vectors, the
// state and state-gradient checkpoints, and the chunk's Y, V' and dV'.
struct BwdWorkspace {
    ChunkWorkspace fwd;
    size_t off_t, off_p, off_gk, off_vec, off_ck, off_ds, off_y, off_vp, off_dvp;
    size_t off_qh, off_kh, off_v32, off_rqk;   // with q/k normalisation: q^, k^, v as fp32, 1/||q||, 1/||k||
    size_t total;
};
BwdWorkspace chunk_bwd_workspace_layout(int32_t B, int32_t T, int32_t N, bool packed, int32_t H, int32_t dk,
                                        int32_t dv, bool qk_norm);
hipError_t launch_chunk_bwd(const ChunkArgs &a, const BwdArgs &g, hipStream_t stream);
// G0 on its own (validates cu_seqlens and builds the chunk-row table).
// With seg_chunks > 0 it also lays out the segment units: seg_first[n] and
// seg_cnt[n] per sequence, seg_tab[2u], seg_tab[2u + 1] = (n, s) per unit, and
// meta[2] = the number of units.
hipError_t launch_chunk_table(int32_t N, int32_t T, const int32_t *cu_seqlens, int32_t *meta, int32_t *cu_ws,
                              int32_t *row0, int32_t *row_tok, int32_t *row_len, int32_t seg_chunks,
                              int32_t *seg_first, int32_t *seg_cnt, int32_t *seg_tab, hipStream_t stream,
                              bool tables = true);   // false: only check cu_seqlens and set meta

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
