// Single-token decode step of the gated delta rule for a batch of resident
// fp32 states, in place (HBM-bound: each state row is read once and written
// once).
//
// Per (sequence n, head h) with S in R^{dv x dk} (row i = value dim i):
//   Sbar = alpha S                       forget first
//   u_i  = beta (v_i - Sbar_i . k)       error of the decayed memory along k
//   S'_i = Sbar_i + u_i k^T              write
//   o_i  = S'_i . q = alpha (S_i . q) + u_i (k . q)
// The ordered form (forget, then correct the decayed error) is the tutorial
// page's statement of the rule; expanding it gives eq. (10) of the Gated
// Delta Networks paper (section 3.1).  The last line reuses S_i . q and
// k . q so o needs no second pass over the row.
//
// Layout: one 256-thread block per (n, h).  DK/8 threads share a state row,
// each holding 8 consecutive fp32 (two 16-byte loads); every thread keeps R
// rows in registers so a block has R * 256 * 32 bytes of loads in flight
// before the first reduction.  Row dot products reduce across the DK/8 lanes
// with xor shuffles inside aligned lane groups.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

// Lane data movement inside a 16-lane DPP row (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7 - i within 8 lanes
constexpr int kDppMirror = 0x140;       // lane i <- lane 15 - i within 16 lanes

// Sum over aligned groups of TPR lanes; every lane of a group gets the same
// bits (each step adds two partial sums that the partner lane adds in the
// other order).
template <int TPR>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(TPR == 1 || TPR == 2 || TPR == 4 || TPR == 8 || TPR == 16 || TPR == 32, "group of 1..32 lanes");
    if constexpr (TPR >= 2) x += dpp_f32<kDppQuadXor1>(x);
    if constexpr (TPR >= 4) x += dpp_f32<kDppQuadXor2>(x);
    if constexpr (TPR >= 8) x += dpp_f32<kDppHalfMirror>(x);
    if constexpr (TPR >= 16) x += dpp_f32<kDppMirror>(x);
    if constexpr (TPR >= 32) x += __shfl_xor(x, 16, 64);
    return x;
}

template <typename in_t, typename out_t, int DK>
__global__ __launch_bounds__(256) void decode_step_kernel(int H, int DV, int qk_norm, float *__restrict__ state,
                                                          const in_t *__restrict__ q,
                                                          const in_t *__restrict__ k,
                                                          const in_t *__restrict__ v,
                                                          const float *__restrict__ log_alpha,
                                                          const float *__restrict__ beta,
                                                          out_t *__restrict__ o) {
    constexpr int TPR = DK / 8;      // threads per state row
    constexpr int RPP = 256 / TPR;   // rows per pass of the block
    constexpr int R = 8;             // rows held per thread
    const int64_t nh = blockIdx.x;
    const int t = threadIdx.x;
    const int sub = t % TPR;
    const int rr = t / TPR;

    float kk[8], qq[8];
    load8_f32(k + nh * DK + sub * 8, kk);
    load8_f32(q + nh * DK + sub * 8, qq);
    if (qk_norm) {
        // q / ||q||, k / ||k|| (an all-zero vector stays zero)
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sk += kk[e] * kk[e];
            sq += qq[e] * qq[e];
        }
        sk = group_sum<TPR>(sk);
        sq = group_sum<TPR>(sq);
        const float rk = sk > 0.f ? rsqrtf(sk) : 0.f, rq = sq > 0.f ? rsqrtf(sq) : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kk[e] *= rk;
            qq[e] *= rq;
        }
    }
    const float a = expf(log_alpha[nh]);
    const float b = beta[nh];
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) kq += kk[e] * qq[e];
    kq = group_sum<TPR>(kq);

    float *S = state + nh * (int64_t)DV * DK;
    const in_t *vv = v + nh * DV;
    out_t *oo = o + nh * DV;

    for (int base = 0; base < DV; base += RPP * R) {
        float4_t s[R][2];
#pragma unroll
        for (int p = 0; p < R; ++p) {
            const int row = base + p * RPP + rr;
            if (row < DV) {
                const float4_t *src = reinterpret_cast<const float4_t *>(S + (int64_t)row * DK + sub * 8);
                s[p][0] = src[0];
                s[p][1] = src[1];
            } else {
                s[p][0] = float4_t{0.f, 0.f, 0.f, 0.f};
                s[p][1] = float4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int p = 0; p < R; ++p) {
            const int row = base + p * RPP + rr;
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sk += s[p][0][e] * kk[e] + s[p][1][e] * kk[4 + e];
                sq += s[p][0][e] * qq[e] + s[p][1][e] * qq[4 + e];
            }
            sk = group_sum<TPR>(sk);
            sq = group_sum<TPR>(sq);
            if (row < DV) {
                const float vi = to_f32(vv[row]);
                const float u = b * (vi - a * sk);
                float4_t n0, n1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    n0[e] = a * s[p][0][e] + u * kk[e];
                    n1[e] = a * s[p][1][e] + u * kk[4 + e];
                }
                float4_t *dst = reinterpret_cast<float4_t *>(S + (int64_t)row * DK + sub * 8);
                dst[0] = n0;
                dst[1] = n1;
                if (sub == 0) oo[row] = from_f32<out_t>(a * sq + u * kq);
            }
        }
    }
}

// Token-serial form of gdn_chunk_fwd for batches of short sequences (a few
// tokens each, e.g. appending to resident states): a 256-thread block holds a
// group of one (sequence, head)'s state rows in registers, steps through the
// sequence's tokens with the decode update above, writes o per token and the
// state once.  The rule is row-separable (row i of S evolves with k, v_i and
// the gates only), so groups of rows evolve with no exchange: blockIdx.y
// picks the row group and a state is spread over several blocks.  Any
// sequence length is handled; the host picks this kernel when the batch
// averages few tokens per sequence.  The initial and final states may be the
// same buffer: each block reads its rows before writing them.
//
// The token loop is VALU-bound, so it is cut to three fused multiply-adds
// per state element and token:
//   * the decay is kept as one block-wide scale c (S = c * Shat): with
//     c' = c alpha, u = beta (v - c' Shat k), Shat += (u / c') k^T and
//     o = c' (Shat q) + u (k . q), all from the rows' dot products before
//     the write.  When c' leaves [2^-64, 2^64] (or alpha is 0) the scale is
//     folded into Shat first and restarts at 1, so Shat stays in range.
//   * k . q (and the optional L2 normalisation of q and k) is computed once
//     per token while staging it, not per row.
//   * each thread holds 16 columns of a row, so a row's dot product reduces
//     over dk / 16 lanes with DPP moves.
// Tokens go through LDS in batches of kShortTB: one cooperative load of k, q,
// the group's v values and the gates per batch, so the token loop itself
// waits on no global memory.
constexpr int kShortTB = 16;
constexpr int kShortEPT = 16;    // state columns per thread and row
constexpr int kShortR = 4;       // rows per thread
constexpr float kScaleLo = 0x1p-64f, kScaleHi = 0x1p64f;

// Rows of one row group of the token-serial kernel.
__host__ __device__ constexpr int short_rows_per_block(int dk) {
    return kShortR * 256 / (dk / (kShortEPT < dk ? kShortEPT : dk));
}

template <typename in_t, typename out_t, int DK>
__global__ __launch_bounds__(256) void chunk_short_kernel(int H, int DV, int T, int qk_norm,
                                                          const int32_t *__restrict__ cu,
                                                          int32_t *__restrict__ meta,
                                                          const in_t *__restrict__ q,
                                                          const in_t *__restrict__ k,
                                                          const in_t *__restrict__ v,
                                                          const float *__restrict__ log_alpha,
                                                          const float *__restrict__ beta,
                                                          const float *init_state, float *final_state,
                                                          out_t *__restrict__ o) {
    constexpr int EPT = kShortEPT < DK ? kShortEPT : DK;
    constexpr int TPR = DK / EPT;    // threads per state row
    constexpr int NV = EPT / 4;      // float4 columns per thread: columns 4 (m TPR + sub) .. +3
    constexpr int RPP = 256 / TPR;   // rows per pass of the block
    constexpr int R = kShortR;
    constexpr int RB = RPP * R;      // rows of one row group
    static_assert(RB == short_rows_per_block(DK), "host and kernel row groups agree");
    constexpr int TB = kShortTB;
    constexpr int STPR = DK / 8;     // staging: threads per token, 8 values each
    constexpr int SRPP = 256 / STPR;
    // One batch of tokens: k and q (fp32, normalised when asked for), the row
    // group's v values, alpha, beta and k . q.
    __shared__ __align__(16) float sk_[TB][DK], sq_[TB][DK], sv_[TB][RB], sa_[TB], sb_[TB], skq_[TB];
    if (cu) {
        if (meta[1] != 0) return;    // cu_seqlens rejected by the table pass: write nothing
    } else if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        meta[0] = (int)(gridDim.x / H) * ((T + kChunk - 1) / kChunk);
        meta[1] = 0;
    }
    const int nh = blockIdx.x, n = nh / H, h = nh % H;
    const int tb = cu ? cu[n] : n * T, te = cu ? cu[n + 1] : (n + 1) * T;
    const int t = threadIdx.x;
    const int sub = t % TPR, rr = t / TPR;
    const int ssub = t % STPR, srr = t / STPR;
    const int64_t sbase = (int64_t)nh * DV * DK;

    // Stage tokens t0 .. t0 + TB - 1 (clipped to the sequence) of the row group at `base`.
    auto stage = [&](int t0, int base) {
        const int nt = min(TB, te - t0);
        __syncthreads();   // the previous batch is no longer read
        for (int tt = srr; tt < nt; tt += SRPP) {
            const int64_t th = (int64_t)(t0 + tt) * H + h;
            float kk[8], qq[8];
            load8_f32(k + th * DK + ssub * 8, kk);
            load8_f32(q + th * DK + ssub * 8, qq);
            if (qk_norm) {
                float a2 = 0.f, b2 = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a2 += kk[e] * kk[e];
                    b2 += qq[e] * qq[e];
                }
                a2 = group_sum<STPR>(a2);
                b2 = group_sum<STPR>(b2);
                const float rk = a2 > 0.f ? rsqrtf(a2) : 0.f, rq = b2 > 0.f ? rsqrtf(b2) : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kk[e] *= rk;
                    qq[e] *= rq;
                }
            }
            float kq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) kq += kk[e] * qq[e];
            kq = group_sum<STPR>(kq);
            *reinterpret_cast<float4_t *>(&sk_[tt][ssub * 8]) = float4_t{kk[0], kk[1], kk[2], kk[3]};
            *reinterpret_cast<float4_t *>(&sk_[tt][ssub * 8 + 4]) = float4_t{kk[4], kk[5], kk[6], kk[7]};
            *reinterpret_cast<float4_t *>(&sq_[tt][ssub * 8]) = float4_t{qq[0], qq[1], qq[2], qq[3]};
            *reinterpret_cast<float4_t *>(&sq_[tt][ssub * 8 + 4]) = float4_t{qq[4], qq[5], qq[6], qq[7]};
            if (ssub == 0) {
                sa_[tt] = expf(log_alpha[th]);
                sb_[tt] = beta[th];
                skq_[tt] = kq;
            }
        }
        for (int i = t; i < nt * RB; i += 256) {
            const int tt = i / RB, row = base + i % RB;
            sv_[tt][i % RB] = row < DV ? to_f32(v[((int64_t)(t0 + tt) * H + h) * DV + row]) : 0.f;
        }
        __syncthreads();
    };

    for (int base = blockIdx.y * RB; base < DV; base += gridDim.y * RB) {
        float4_t s[R][NV];
#pragma unroll
        for (int p = 0; p < R; ++p) {
            const int row = base + p * RPP + rr;
#pragma unroll
            for (int m = 0; m < NV; ++m)
                s[p][m] = (row < DV && init_state)
                              ? *reinterpret_cast<const float4_t *>(init_state + sbase + (int64_t)row * DK +
                                                                    4 * (m * TPR + sub))
                              : float4_t{0.f, 0.f, 0.f, 0.f};
        }
        int staged = -1;
        float c = 1.f;   // S = c * s for this block's rows
        for (int t0 = tb; t0 < te; t0 += TB) {
            if (staged != t0) {
                stage(t0, base);
                staged = t0;
            }
            const int nt = min(TB, te - t0);
            for (int tt = 0; tt < nt; ++tt) {
                float cn = c * sa_[tt];
                if (!(cn >= kScaleLo && cn <= kScaleHi)) {   // block-uniform
#pragma unroll
                    for (int p = 0; p < R; ++p)
#pragma unroll
                        for (int m = 0; m < NV; ++m) s[p][m] *= cn;
                    cn = 1.f;
                }
                c = cn;
                const float rc = __builtin_amdgcn_rcpf(cn), b = sb_[tt], kq = skq_[tt];
                float4_t kv[NV];
                float dk_[R], dq_[R];
#pragma unroll
                for (int m = 0; m < NV; ++m) {
                    kv[m] = *reinterpret_cast<const float4_t *>(&sk_[tt][4 * (m * TPR + sub)]);
                    const float4_t qv = *reinterpret_cast<const float4_t *>(&sq_[tt][4 * (m * TPR + sub)]);
#pragma unroll
                    for (int j = 0; j < R; ++j) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (m == 0 && e == 0) {
                                dk_[j] = s[j][0][0] * kv[0][0];
                                dq_[j] = s[j][0][0] * qv[0];
                            } else {
                                dk_[j] = fmaf(s[j][m][e], kv[m][e], dk_[j]);
                                dq_[j] = fmaf(s[j][m][e], qv[e], dq_[j]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    dk_[j] = group_sum<TPR>(dk_[j]);
                    dq_[j] = group_sum<TPR>(dq_[j]);
                }
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const float u = b * (sv_[tt][j * RPP + rr] - cn * dk_[j]);
                    const float w = u * rc;
#pragma unroll
                    for (int m = 0; m < NV; ++m)
#pragma unroll
                        for (int e = 0; e < 4; ++e) s[j][m][e] = fmaf(w, kv[m][e], s[j][m][e]);
                    dq_[j] = cn * dq_[j] + u * kq;
                }
                if (sub == 0) {
                    out_t *oo = o + ((int64_t)(t0 + tt) * H + h) * DV;
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        const int row = base + j * RPP + rr;
                        if (row < DV) oo[row] = from_f32<out_t>(dq_[j]);
                    }
                }
            }
        }
        if (final_state) {
#pragma unroll
            for (int p = 0; p < R; ++p) {
                const int row = base + p * RPP + rr;
                if (row < DV) {
#pragma unroll
                    for (int m = 0; m < NV; ++m)
                        *reinterpret_cast<float4_t *>(final_state + sbase + (int64_t)row * DK +
                                                      4 * (m * TPR + sub)) = c * s[p][m];
                }
            }
        }
    }
}

template <typename in_t, typename out_t>
static hipError_t short_dispatch_dk(const ChunkArgs &a, int32_t *meta, hipStream_t st) {
    const int rb = short_rows_per_block(a.dk);
    const dim3 grid((unsigned)((int64_t)a.N * a.H), (unsigned)((a.dv + rb - 1) / rb)), block(256);
    auto *q = static_cast<const in_t *>(a.q);
    auto *k = static_cast<const in_t *>(a.k);
    auto *v = static_cast<const in_t *>(a.v);
    auto *o = static_cast<out_t *>(a.o);
    const int qn = (a.flags & kFlagQkL2Norm) ? 1 : 0;
    ProfScope prof("gdn_chunk_short", st);
    switch (a.dk) {
    case 32:
        chunk_short_kernel<in_t, out_t, 32><<<grid, block, 0, st>>>(a.H, a.dv, a.T, qn, a.cu_seqlens, meta, q, k, v,
                                                                  a.log_alpha, a.beta, a.init_state, a.final_state, o);
        break;
    case 64:
        chunk_short_kernel<in_t, out_t, 64><<<grid, block, 0, st>>>(a.H, a.dv, a.T, qn, a.cu_seqlens, meta, q, k, v,
                                                                  a.log_alpha, a.beta, a.init_state, a.final_state, o);
        break;
    case 128:
        chunk_short_kernel<in_t, out_t, 128><<<grid, block, 0, st>>>(a.H, a.dv, a.T, qn, a.cu_seqlens, meta, q, k, v,
                                                                   a.log_alpha, a.beta, a.init_state, a.final_state, o);
        break;
    case 256:
        chunk_short_kernel<in_t, out_t, 256><<<grid, block, 0, st>>>(a.H, a.dv, a.T, qn, a.cu_seqlens, meta, q, k, v,
                                                                   a.log_alpha, a.beta, a.init_state, a.final_state, o);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename in_t>
static hipError_t short_dispatch_out(const ChunkArgs &a, int32_t *meta, hipStream_t st) {
    switch (a.out_dtype) {
    case DT_FP32: return short_dispatch_dk<in_t, float>(a, meta, st);
    case DT_BF16: return short_dispatch_dk<in_t, bf16_t>(a, meta, st);
    case DT_FP16: return short_dispatch_dk<in_t, _Float16>(a, meta, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_short(const ChunkArgs &a, int32_t *meta, hipStream_t st) {
    if ((int64_t)a.N * a.H == 0) return hipSuccess;
    switch (a.in_dtype) {
    case DT_FP32: return short_dispatch_out<float>(a, meta, st);
    case DT_BF16: return short_dispatch_out<bf16_t>(a, meta, st);
    case DT_FP16: return short_dispatch_out<_Float16>(a, meta, st);
    }
    return hipErrorInvalidValue;
}

template <typename in_t, typename out_t>
static hipError_t decode_dispatch_dk(const DecodeArgs &d, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)d.N * d.H)), block(256);
    auto *q = static_cast<const in_t *>(d.q);
    auto *k = static_cast<const in_t *>(d.k);
    auto *v = static_cast<const in_t *>(d.v);
    auto *o = static_cast<out_t *>(d.o);
    ProfScope prof("gdn_decode_step", st);
    switch (d.dk) {
    case 32:
        decode_step_kernel<in_t, out_t, 32><<<grid, block, 0, st>>>(d.H, d.dv, (d.flags & kFlagQkL2Norm) ? 1 : 0, d.state, q, k, v, d.log_alpha, d.beta, o);
        break;
    case 64:
        decode_step_kernel<in_t, out_t, 64><<<grid, block, 0, st>>>(d.H, d.dv, (d.flags & kFlagQkL2Norm) ? 1 : 0, d.state, q, k, v, d.log_alpha, d.beta, o);
        break;
    case 128:
        decode_step_kernel<in_t, out_t, 128><<<grid, block, 0, st>>>(d.H, d.dv, (d.flags & kFlagQkL2Norm) ? 1 : 0, d.state, q, k, v, d.log_alpha, d.beta, o);
        break;
    case 256:
        decode_step_kernel<in_t, out_t, 256><<<grid, block, 0, st>>>(d.H, d.dv, (d.flags & kFlagQkL2Norm) ? 1 : 0, d.state, q, k, v, d.log_alpha, d.beta, o);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename in_t>
static hipError_t decode_dispatch_out(const DecodeArgs &d, hipStream_t st) {
    switch (d.out_dtype) {
    case DT_FP32: return decode_dispatch_dk<in_t, float>(d, st);
    case DT_BF16: return decode_dispatch_dk<in_t, bf16_t>(d, st);
    case DT_FP16: return decode_dispatch_dk<in_t, _Float16>(d, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_step(const DecodeArgs &d, hipStream_t st) {
    if ((int64_t)d.N * d.H == 0) return hipSuccess;
    switch (d.in_dtype) {
    case DT_FP32: return decode_dispatch_out<float>(d, st);
    case DT_BF16: return decode_dispatch_out<bf16_t>(d, st);
    case DT_FP16: return decode_dispatch_out<_Float16>(d, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
