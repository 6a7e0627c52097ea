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

template <int TPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
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
