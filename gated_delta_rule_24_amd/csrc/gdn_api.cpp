// C ABI of the gated delta rule core: argument validation, workspace sizing,
// launch timing, error reporting.  Declarations and the full contract are in
// include/gdn.h.  Every check runs before anything is enqueued.
#include "gdn.h"
#include "gdn_launch.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

gdn_status ok() {
    g_last_error.clear();
    return GDN_OK;
}

bool valid_dtype(int32_t d) { return d == GDN_FP32 || d == GDN_BF16 || d == GDN_FP16; }
size_t dtype_size(int32_t d) { return d == GDN_FP32 ? 4 : 2; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Range {
    const char *name;
    uintptr_t lo, hi;   // [lo, hi)
};
Range rng(const char *name, const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}
bool overlap(const Range &a, const Range &b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

gdn_status hip_fail(hipError_t e, const char *what) {
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- launch timing ------------------------------------------------------------
struct ProfRecord {
    const char *name;
    hipEvent_t begin, end;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof_records;

void prof_clear_locked() {
    for (auto &r : g_prof_records) {
        hipEventDestroy(r.begin);
        hipEventDestroy(r.end);
    }
    g_prof_records.clear();
}

static_assert(gdn::kFlagQkL2Norm == GDN_QK_L2NORM, "flag values");

gdn_status check_chunk_desc(const gdn_chunk_desc *d) {
    if (!d) return fail(GDN_ERR_NULL, "desc is NULL");
    if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype))
        return fail(GDN_ERR_DTYPE, "unknown dtype code (in %d, out %d)", d->in_dtype, d->out_dtype);
    if (d->batch < 1 || d->seqlen < 0 || d->heads < 1 || d->num_seqs < 1)
        return fail(GDN_ERR_SHAPE, "need batch >= 1, seqlen >= 0, heads >= 1, num_seqs >= 1 (got %d, %d, %d, %d)",
                    d->batch, d->seqlen, d->heads, d->num_seqs);
    if ((int64_t)d->batch * d->seqlen > INT32_MAX / 2)
        return fail(GDN_ERR_SHAPE, "batch * seqlen too large");
    if (d->dk <= 0 || d->dv <= 0) return fail(GDN_ERR_SHAPE, "head dims must be positive");
    if (d->chunk != gdn::kChunk)
        return fail(GDN_ERR_UNSUPPORTED, "chunk %d not built (supported: %d)", d->chunk, gdn::kChunk);
    const bool dk_ok = d->dk == 32 || d->dk == 64 || d->dk == 128 || (d->dk == 256 && d->in_dtype != GDN_FP32);
    if (!dk_ok) return fail(GDN_ERR_UNSUPPORTED, "dk %d not built for this input dtype", d->dk);
    if (d->dv % 16 != 0 || d->dv > 1024)
        return fail(GDN_ERR_UNSUPPORTED, "dv %d not built (multiple of 16, at most 1024)", d->dv);
    if (d->flags & ~GDN_QK_L2NORM) return fail(GDN_ERR_UNSUPPORTED, "unknown flags 0x%x", d->flags);
    return GDN_OK;
}

}  // namespace

namespace gdn {

ProfScope::ProfScope(const char *name, hipStream_t stream) : name_(name), stream_(stream), begin_(nullptr) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return;
    hipEventRecord(e, stream);
    begin_ = e;
}

ProfScope::~ProfScope() {
    if (!begin_) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
        hipEventDestroy(static_cast<hipEvent_t>(begin_));
        return;
    }
    hipEventRecord(e, stream_);
    g_prof_records.push_back(ProfRecord{name_, static_cast<hipEvent_t>(begin_), e});
}

}  // namespace gdn

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_string(gdn_status s) {
    switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS";
    case GDN_ERR_DEVICE_INPUT: return "GDN_ERR_DEVICE_INPUT";
    }
    return "GDN_ERR_UNKNOWN";
}

const char *gdn_last_error_message(void) { return g_last_error.c_str(); }

gdn_status gdn_chunk_fwd_workspace_size(const gdn_chunk_desc *desc, size_t *bytes) {
    if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
    gdn_status s = check_chunk_desc(desc);
    if (s != GDN_OK) return s;
    // Size for the larger of the packed and batched layouts, so the answer
    // does not depend on whether cu_seqlens is passed later.
    const auto a = gdn::chunk_workspace_layout(desc->batch, desc->seqlen, desc->num_seqs, true,
                                               desc->heads, desc->in_dtype, desc->dk, desc->dv);
    const auto b = gdn::chunk_workspace_layout(desc->batch, desc->seqlen, desc->num_seqs, false,
                                               desc->heads, desc->in_dtype, desc->dk, desc->dv);
    *bytes = a.total > b.total ? a.total : b.total;
    return ok();
}

static gdn_status chunk_fwd_impl(const gdn_chunk_desc *desc, const void *q, const void *k, const void *v,
                                 const float *log_alpha, const float *beta, const float *init_state,
                                 const int32_t *cu_seqlens, void *o, float *final_state, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream, const char *ws_name) {
    gdn_status s = check_chunk_desc(desc);
    if (s != GDN_OK) return s;
    const gdn_chunk_desc &d = *desc;
    const bool packed = cu_seqlens != nullptr;
    if (packed && d.batch != 1) return fail(GDN_ERR_SHAPE, "cu_seqlens requires batch == 1 (got %d)", d.batch);
    if (!packed && d.num_seqs != d.batch)
        return fail(GDN_ERR_SHAPE, "without cu_seqlens num_seqs must equal batch (%d != %d)", d.num_seqs, d.batch);
    const int64_t toks = (int64_t)d.batch * d.seqlen;
    if (toks > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
        return fail(GDN_ERR_NULL, "q, k, v, log_alpha, beta and o are required");
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL");
    const auto w = gdn::chunk_workspace_layout(d.batch, d.seqlen, d.num_seqs, packed, d.heads, d.in_dtype, d.dk,
                                               d.dv);
    if (workspace_bytes < w.total)
        return fail(GDN_ERR_WORKSPACE, "%s has %zu bytes, this call needs %zu", ws_name, workspace_bytes, w.total);
    const void *ptrs[] = {q, k, v, init_state, o, final_state, workspace};
    const char *names[] = {"q", "k", "v", "init_state", "o", "final_state", "workspace"};
    for (int i = 0; i < 7; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(GDN_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const void *sptrs[] = {log_alpha, beta, cu_seqlens};
    const char *snames[] = {"log_alpha", "beta", "cu_seqlens"};
    for (int i = 0; i < 3; ++i)
        if (sptrs[i] && !aligned4(sptrs[i])) return fail(GDN_ERR_ALIGN, "%s is not 4-byte aligned", snames[i]);

    const size_t isz = dtype_size(d.in_dtype), osz = dtype_size(d.out_dtype);
    const size_t th = (size_t)toks * d.heads;
    const size_t state_bytes = sizeof(float) * (size_t)d.num_seqs * d.heads * d.dv * d.dk;
    const Range r_o = rng("o", o, th * d.dv * osz);
    const Range ins[] = {rng("q", q, th * d.dk * isz), rng("k", k, th * d.dk * isz), rng("v", v, th * d.dv * isz),
                         rng("log_alpha", log_alpha, th * 4), rng("beta", beta, th * 4),
                         rng("init_state", init_state, state_bytes),
                         rng("cu_seqlens", cu_seqlens, sizeof(int32_t) * (d.num_seqs + 1)),
                         rng("final_state", final_state, state_bytes), rng("workspace", workspace, w.total)};
    for (const Range &r : ins)
        if (overlap(r_o, r)) return fail(GDN_ERR_ALIAS, "o overlaps %s", r.name);
    if (final_state && init_state && final_state != init_state &&
        overlap(rng("final_state", final_state, state_bytes), rng("init_state", init_state, state_bytes)))
        return fail(GDN_ERR_ALIAS, "final_state partially overlaps init_state");
    const Range r_ws = rng("workspace", workspace, w.total);
    for (int i = 0; i < 8; ++i)
        if (overlap(r_ws, ins[i])) return fail(GDN_ERR_ALIAS, "workspace overlaps %s", ins[i].name);

    gdn::ChunkArgs a{d.batch, d.seqlen, d.heads, d.dk, d.dv, d.num_seqs, d.in_dtype, d.out_dtype, d.flags,
                     q, k, v, log_alpha, beta, init_state, cu_seqlens, o, final_state, workspace};
    hipError_t e = gdn::launch_chunk_fwd(a, stream);
    if (e != hipSuccess) return hip_fail(e, "gdn_chunk_fwd launch");
    return ok();
}

gdn_status gdn_chunk_fwd(const gdn_chunk_desc *desc, const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *beta, const float *init_state,
                         const int32_t *cu_seqlens, void *o, float *final_state, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    return chunk_fwd_impl(desc, q, k, v, log_alpha, beta, init_state, cu_seqlens, o, final_state, workspace,
                          workspace_bytes, stream, "workspace");
}

// ---- gdn_chunk_fwd without a caller workspace -----------------------------------
// The workspace of gdn_chunk_fwd_noalloc is this array: one copy per GPU,
// allocated when the code object is loaded and held until the process ends.
// Its name is only a host-side handle; the device address of the current
// GPU's copy comes from hipGetSymbolAddress, looked up once per device on the
// first call made with that device current and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static gdn_status scratch_for_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return GDN_OK;
}

gdn_status gdn_chunk_fwd_noalloc(const gdn_chunk_desc *desc, const void *q, const void *k, const void *v,
                                 const float *log_alpha, const float *beta, const float *init_state,
                                 const int32_t *cu_seqlens, void *o, float *final_state, hipStream_t stream) {
    // The size limit is checked first, on the host, so an oversized call
    // fails the same way with or without a GPU.
    gdn_status s = check_chunk_desc(desc);
    if (s != GDN_OK) return s;
    const auto w = gdn::chunk_workspace_layout(desc->batch, desc->seqlen, desc->num_seqs, cu_seqlens != nullptr,
                                               desc->heads, desc->in_dtype, desc->dk, desc->dv);
    if (w.total > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
        return fail(GDN_ERR_WORKSPACE,
                    "this call needs %zu bytes of workspace, more than the %zu-byte scratch array of "
                    "gdn_chunk_fwd_noalloc; use gdn_chunk_fwd with a workspace",
                    w.total, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    s = scratch_for_current_device(&ws);
    if (s != GDN_OK) return s;
    return chunk_fwd_impl(desc, q, k, v, log_alpha, beta, init_state, cu_seqlens, o, final_state, ws,
                          (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream, "the no-allocation scratch array");
}

gdn_status gdn_chunk_bwd_workspace_size(const gdn_chunk_desc *desc, size_t *bytes) {
    if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
    gdn_status s = check_chunk_desc(desc);
    if (s != GDN_OK) return s;
    const bool qk_norm = (desc->flags & GDN_QK_L2NORM) != 0;
    const auto a = gdn::chunk_bwd_workspace_layout(desc->batch, desc->seqlen, desc->num_seqs, true, desc->heads,
                                                   desc->dk, desc->dv, qk_norm);
    const auto b = gdn::chunk_bwd_workspace_layout(desc->batch, desc->seqlen, desc->num_seqs, false, desc->heads,
                                                   desc->dk, desc->dv, qk_norm);
    *bytes = a.total > b.total ? a.total : b.total;
    return ok();
}

gdn_status gdn_chunk_bwd(const gdn_chunk_desc *desc, const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *beta, const float *init_state,
                         const int32_t *cu_seqlens, const float *d_o, const float *d_final_state, float *dq,
                         float *dk, float *dv, float *dlog_alpha, float *dbeta, float *d_init_state,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
    gdn_status s = check_chunk_desc(desc);
    if (s != GDN_OK) return s;
    const gdn_chunk_desc &d = *desc;
    if (d.dk > 128) return fail(GDN_ERR_UNSUPPORTED, "dk %d not built for the backward pass (at most 128)", d.dk);
    const bool packed = cu_seqlens != nullptr;
    if (packed && d.batch != 1) return fail(GDN_ERR_SHAPE, "cu_seqlens requires batch == 1 (got %d)", d.batch);
    if (!packed && d.num_seqs != d.batch)
        return fail(GDN_ERR_SHAPE, "without cu_seqlens num_seqs must equal batch (%d != %d)", d.num_seqs, d.batch);
    const int64_t toks = (int64_t)d.batch * d.seqlen;
    if (toks > 0 && (!q || !k || !v || !log_alpha || !beta || !d_o || !dq || !dk || !dv || !dlog_alpha || !dbeta))
        return fail(GDN_ERR_NULL, "q, k, v, log_alpha, beta, d_o, dq, dk, dv, dlog_alpha and dbeta are required");
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL");
    const auto w = gdn::chunk_bwd_workspace_layout(d.batch, d.seqlen, d.num_seqs, packed, d.heads, d.dk, d.dv,
                                                   (d.flags & GDN_QK_L2NORM) != 0);
    if (workspace_bytes < w.total)
        return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, w.total);
    const void *ptrs[] = {q, k, v, init_state, d_o, d_final_state, dq, dk, dv, d_init_state, workspace};
    const char *names[] = {"q", "k", "v", "init_state", "d_o", "d_final_state", "dq", "dk", "dv", "d_init_state",
                           "workspace"};
    for (int i = 0; i < 11; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(GDN_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const void *sptrs[] = {log_alpha, beta, cu_seqlens, dlog_alpha, dbeta};
    const char *snames[] = {"log_alpha", "beta", "cu_seqlens", "dlog_alpha", "dbeta"};
    for (int i = 0; i < 5; ++i)
        if (sptrs[i] && !aligned4(sptrs[i])) return fail(GDN_ERR_ALIGN, "%s is not 4-byte aligned", snames[i]);

    const size_t isz = dtype_size(d.in_dtype);
    const size_t th = (size_t)toks * d.heads;
    const size_t state_bytes = sizeof(float) * (size_t)d.num_seqs * d.heads * d.dv * d.dk;
    const Range ins[] = {rng("q", q, th * d.dk * isz), rng("k", k, th * d.dk * isz), rng("v", v, th * d.dv * isz),
                         rng("log_alpha", log_alpha, th * 4), rng("beta", beta, th * 4),
                         rng("init_state", init_state, state_bytes),
                         rng("cu_seqlens", cu_seqlens, sizeof(int32_t) * (d.num_seqs + 1)),
                         rng("d_o", d_o, th * d.dv * 4), rng("d_final_state", d_final_state, state_bytes)};
    const Range outs[] = {rng("dq", dq, th * d.dk * 4), rng("dk", dk, th * d.dk * 4), rng("dv", dv, th * d.dv * 4),
                          rng("dlog_alpha", dlog_alpha, th * 4), rng("dbeta", dbeta, th * 4),
                          rng("d_init_state", d_init_state, state_bytes), rng("workspace", workspace, w.total)};
    for (int i = 0; i < 7; ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r)) return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[i].name, r.name);
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], outs[j])) return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
    }

    gdn::ChunkArgs a{d.batch, d.seqlen, d.heads, d.dk, d.dv, d.num_seqs, d.in_dtype, d.out_dtype, d.flags,
                     q, k, v, log_alpha, beta, init_state, cu_seqlens, nullptr, nullptr, workspace};
    gdn::BwdArgs g{d_o, d_final_state, dq, dk, dv, dlog_alpha, dbeta, d_init_state};
    hipError_t e = gdn::launch_chunk_bwd(a, g, stream);
    if (e != hipSuccess) return hip_fail(e, "gdn_chunk_bwd launch");
    return ok();
}

gdn_status gdn_chunk_fwd_check(const void *workspace, hipStream_t stream, int32_t *code) {
    if (!workspace || !code) return fail(GDN_ERR_NULL, "workspace and code are required");
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int32_t meta[2] = {0, 0};
    e = hipMemcpy(meta, workspace, sizeof(meta), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
    *code = meta[1];
    if (meta[1] != 0) return fail(GDN_ERR_DEVICE_INPUT, "cu_seqlens rejected on the device (code %d)", meta[1]);
    return ok();
}

gdn_status gdn_decode_step(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t in_dtype, int32_t out_dtype,
                           int32_t flags, float *state, const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, void *o, hipStream_t stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return fail(GDN_ERR_DTYPE, "unknown dtype code (in %d, out %d)", in_dtype, out_dtype);
    if (N < 0 || H < 1 || dv < 1) return fail(GDN_ERR_SHAPE, "need N >= 0, H >= 1, dv >= 1");
    if (dv > 4096) return fail(GDN_ERR_UNSUPPORTED, "dv %d not built (at most 4096)", dv);
    if (!(dk == 32 || dk == 64 || dk == 128 || dk == 256))
        return fail(GDN_ERR_UNSUPPORTED, "dk %d not built (32, 64, 128, 256)", dk);
    if (flags & ~GDN_QK_L2NORM) return fail(GDN_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    if ((int64_t)N * H > INT32_MAX) return fail(GDN_ERR_SHAPE, "N * H too large");
    if ((int64_t)N * H == 0) return ok();
    if (!state || !q || !k || !v || !log_alpha || !beta || !o)
        return fail(GDN_ERR_NULL, "state, q, k, v, log_alpha, beta and o are required");
    const void *ptrs[] = {state, q, k, v, o};
    const char *names[] = {"state", "q", "k", "v", "o"};
    for (int i = 0; i < 5; ++i)
        if (!aligned16(ptrs[i])) return fail(GDN_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    if (!aligned4(log_alpha) || !aligned4(beta)) return fail(GDN_ERR_ALIGN, "log_alpha and beta must be 4-byte aligned");
    const size_t nh = (size_t)N * H;
    const Range r_o = rng("o", o, nh * dv * dtype_size(out_dtype));
    const Range others[] = {rng("state", state, nh * dv * dk * sizeof(float)), rng("q", q, nh * dk * dtype_size(in_dtype)),
                            rng("k", k, nh * dk * dtype_size(in_dtype)), rng("v", v, nh * dv * dtype_size(in_dtype)),
                            rng("log_alpha", log_alpha, nh * 4), rng("beta", beta, nh * 4)};
    for (const Range &r : others)
        if (overlap(r_o, r)) return fail(GDN_ERR_ALIAS, "o overlaps %s", r.name);
    for (int i = 1; i < 6; ++i)
        if (overlap(others[0], others[i])) return fail(GDN_ERR_ALIAS, "state overlaps %s", others[i].name);
    gdn::DecodeArgs a{N, H, dk, dv, in_dtype, out_dtype, flags, state, q, k, v, log_alpha, beta, o};
    hipError_t e = gdn::launch_decode_step(a, stream);
    if (e != hipSuccess) return hip_fail(e, "gdn_decode_step launch");
    return ok();
}

gdn_status gdn_profile_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (on) prof_clear_locked();
    g_prof_on = on != 0;
    return ok();
}

namespace {
struct ProfSummary {
    const char *name;
    int64_t launches;
    double ms;
};
std::vector<ProfSummary> g_prof_summary;

gdn_status summarise_locked() {
    std::vector<ProfSummary> out;
    for (auto &r : g_prof_records) {
        hipError_t e = hipEventSynchronize(r.end);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, r.begin, r.end);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        bool found = false;
        for (auto &s : out)
            if (strcmp(s.name, r.name) == 0) {
                s.launches += 1;
                s.ms += ms;
                found = true;
            }
        if (!found) out.push_back(ProfSummary{r.name, 1, ms});
    }
    g_prof_summary = out;
    return GDN_OK;
}
}  // namespace

gdn_status gdn_profile_count(int32_t *count) {
    if (!count) return fail(GDN_ERR_NULL, "count is NULL");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    gdn_status s = summarise_locked();
    if (s != GDN_OK) return s;
    *count = (int32_t)g_prof_summary.size();
    return ok();
}

gdn_status gdn_profile_read(int32_t index, const char **name, int64_t *launches, double *total_ms) {
    if (!name || !launches || !total_ms) return fail(GDN_ERR_NULL, "outputs are required");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    gdn_status s = summarise_locked();
    if (s != GDN_OK) return s;
    if (index < 0 || index >= (int32_t)g_prof_summary.size())
        return fail(GDN_ERR_SHAPE, "profile index %d out of range", index);
    *name = g_prof_summary[index].name;
    *launches = g_prof_summary[index].launches;
    *total_ms = g_prof_summary[index].ms;
    return ok();
}

}  // extern "C"
