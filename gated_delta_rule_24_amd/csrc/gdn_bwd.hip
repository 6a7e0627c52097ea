// Backward pass of the chunked gated delta rule: gradients of o and of the
// final state flowing back to q, k, v, log alpha, beta and the initial state.
//
// The pages call the chunkwise algorithm a training method (Gated Delta
// Networks paper, section 3.3, "Hardware-efficient chunkwise training") but
// print no gradient formulas, so these follow from differentiating the chunk
// equations the forward kernels evaluate.  Per chunk, with S the state at
// the chunk start (dv x dk), g the in-chunk cumulative log decay, gamma = e^g,
// kappa_r = e^{g_last - g_r}, Gamma_ri = e^{g_r - g_i} (i <= r):
//
//   forward   A = strictLower(diag(beta)(Gamma o K K^T)),  T = (I + A)^{-1},  M = T diag(beta)
//             P = (Q K^T) o Gamma
//             X = K S^T,  Y = V - diag(gamma) X,  V' = M Y
//             O = diag(gamma) Q S^T + P V'
//             S_next = gamma_last S + V'^T diag(kappa) K
//
//   reverse   (dO, dS_next given; dS flows to the previous chunk)
//             dV' = P^T dO + diag(kappa) K dS_next^T
//             dY  = M^T dV'                    = dV
//             dS  = gamma_last dS_next + dO^T diag(gamma) Q - dY^T diag(gamma) K
//             dP  = lower(dO V'^T),  dM = dV' Y^T,  dT = dM diag(beta),  dA = -T^T dT T^T
//             dbeta_r = sum_x dM_xr T_xr + sum_{i<r} dA_ri Gamma_ri (K K^T)_ri
//             dQ  = diag(gamma) dO S + (dP o Gamma) K
//             dK  = -diag(gamma) dY S + diag(kappa) V' dS_next + (dP o Gamma)^T Q + (dK o + dK o^T) K,
//                   dK o = strictLower(diag(beta) dA o Gamma)
//             dlog alpha_i = sum_{r>=i} dg_r (g is the in-chunk cumulative sum), which
//                   expands to sum_{r>=i} gamma_r dgamma_r + sum_{r<i} kappa_r dkappa_r
//                   + gamma_last <dS_next, S> + sum_{r>=i, c<i} (dGamma o Gamma)_rc,
//                   with dGamma = dP o Q K^T + diag(beta) dA o K K^T,
//                   dgamma_r = dO_r . (Q S^T)_r - dY_r . X_r, dkappa_r = V'_r . (K dS_next^T)_r.
//
// Four kernels:
//   B1 bwd_prep_kernel      per (chunk row, head): g, gamma, kappa, T, P and G = (K K^T) o Gamma.
//   B2 bwd_fwd_pass_kernel  per (sequence, head, 16 value columns), four waves, chunks in order:
//                           replays the state pass and stores the state at every
//                           chunk start (the checkpoints).
//   B3 bwd_rev_pass_kernel  per (sequence, head, two 16-column tiles), chunks in reverse:
//                           the gradient of the state at every chunk end, and of
//                           the initial state.
//   B4 bwd_grad_kernel      per (chunk row, head): every per-token gradient of the
//                           chunk from its checkpoint and state gradient.  One
//                           block per resident slot steps through the items and
//                           loads the next item's first operands during the
//                           current item's last steps.
// B2 also stores each chunk's Y and V', B3 its dV' and dY (= dV, written to
// the output), so B4 recomputes none of the state products.  Y, V' and dV'
// are kept block-major, [item][DV / 16][C][16], so that each 16-column block
// B4 loads is one contiguous run of whole cache lines.
// All arithmetic has fp32 precision, so the gradients carry the same precision
// for every input dtype: products run on the fp32 matrix-core instruction,
// except those with q or k as a factor, which take the 16-bit instruction when
// that is exact (the Gram products of 16-bit q and k in B1; for bf16 inputs the
// products of q or k with an fp32 factor split exactly into three bf16 terms,
// see SplitState).  Matrix-core
// tiles use the lane convention of gdn_device.h: lane l, n = l % 16,
// j = l / 16; an accumulator holds X[4j + i][n]; on issue i of a k-tile kt
// lane (n, j) supplies A[n][16 kt + 4j + i] and B[16 kt + 4j + i][n].
#include <algorithm>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int C = kChunk;

__device__ __forceinline__ void mfma4(float4_t &acc, float a, float b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Sum over the 16 lanes of a DPP row (lanes 16 j .. 16 j + 15); every lane
// of the row gets the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);   // half-row mirror
    x += dpp_mov<0x140>(x);   // row mirror
    return x;
}

__device__ __forceinline__ float4_t zero4() { return float4_t{0.f, 0.f, 0.f, 0.f}; }

// First chunk row, first token and token count of sequence n.
__device__ __forceinline__ void seq_rows(int n, int T, int cpr, const int32_t *cu_ws, const int32_t *row0, int &r0,
                                         int &nrows) {
    if (cpr) {
        r0 = n * cpr;
        nrows = (T + C - 1) / C;
    } else {
        r0 = row0[n];
        nrows = (cu_ws[n + 1] - cu_ws[n] + C - 1) / C;
    }
}

// Per-(row, head) vectors written by B1, in floats from the item's base:
//   [0, C) g,  [C, 2C) gamma,  [2C, 3C) kappa,  [3C, 4C) beta (0 past the row's end).
constexpr int kVecFloats = 4 * C;

}  // namespace

// ============================================================================
// B1: g, gamma, kappa, T = (I + A)^{-1}, P and G per (chunk row, head).
// One wave per item.  The Q and K rows stay in registers as matrix-core
// operands: 16-bit rows on their 16x16x32 instruction (the product of two
// 16-bit values is exact in fp32 and the sums are fp32, so this is the fp32
// Gram matrix), fp32 rows on 16x16x4.  Lane (n, j) holds elements
// 32 p + 8 j .. + 7 of rows 16 b + n, so the accumulator of lower tile (a, b)
// holds row 16 a + n, columns 16 b + 4 j .. + 3: every row of P, G and T
// leaves as 16-byte stores.
//
// T blockwise.  The diagonal 16 x 16 blocks by substitution: T_aa (I + N_a)
// = I gives row n of T_aa from its own later entries and the columns of N_a
// (the strictly lower part of A_aa), so lane (n, j) solves row n of T_jj
// alone.  The others by distance from the diagonal:
//   T_ab = T_aa W,  W = sum_{b <= m < a} (-A_am) T_mb,
// on the matrix cores.  A 16 x 16 block X is held as R(X) (lane (n, j):
// X[n][4j .. 4j + 3]) or C(X) (lane (n, j): X[4j .. 4j + 3][n], the
// accumulator layout); C(X Y) = mm(R(X), C(Y)) and R(X Y) = mm(C(Y), R(X)).
// ============================================================================

// Register passes over dk: the raw Q and K rows of one pass take at most 128
// registers per lane.
template <typename in_t, int DK>
struct BwdPrepShape {
    static constexpr int KPAIR = DK / 32;                                // 32-wide k slices
    static constexpr int REGS = KPAIR * 8 * (int)sizeof(Raw8<in_t>) / 4;  // Q and K, 4 row blocks
    static constexpr int NPASS = REGS > 128 ? REGS / 128 : 1;
    static constexpr int PP = KPAIR / NPASS;
    static_assert(PP * NPASS == KPAIR, "dk splits evenly into passes");
};

template <typename in_t, int DK>
__global__ __launch_bounds__(64) void bwd_prep_kernel(int H, int T, int cpr, int urows,
                                                      const int32_t *__restrict__ meta,
                                                      const int32_t *__restrict__ row_tok,
                                                      const int32_t *__restrict__ row_len,
                                                      const in_t *__restrict__ q, const in_t *__restrict__ k,
                                                      const float *__restrict__ log_alpha,
                                                      const float *__restrict__ beta, float *__restrict__ ws_t,
                                                      float *__restrict__ ws_p, float *__restrict__ ws_g,
                                                      float *__restrict__ ws_vec) {
    using Sh = BwdPrepShape<in_t, DK>;
    constexpr int PP = Sh::PP, NPASS = Sh::NPASS;
    constexpr int BP = 20, BS = 16 * BP + 4;   // one 16 x 16 block in LDS (row pitch, block pitch)
    __shared__ __align__(16) float lds[2 * C + 4 * BS];
    float *sg = lds, *sb = lds + C, *blk = lds + 2 * C;
    if (!cpr && meta[1] != 0) return;   // malformed cu_seqlens: nothing is written
    const int nrows = cpr ? urows : meta[0];
    const int item = blockIdx.x, row = item / H, h = item % H;
    if (row >= nrows) return;
    int tok0, len;
    row_span(row, T, cpr, row_tok, row_len, tok0, len);
    const int l = threadIdx.x, nn = l & 15, jj = l >> 4;

    // Rows past the end of the sequence: log alpha = beta = 0 and zero Q, K
    // rows, inert in every product, and g stays flat there.
    Raw8<in_t> kr[4][PP], qr[4][PP];
    auto load = [&](int s) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int r = 16 * b + nn;
#pragma unroll
            for (int p = 0; p < PP; ++p) {
                if (r < len) {
                    const int64_t off = ((int64_t)(tok0 + r) * H + h) * DK + 32 * (s * PP + p) + 8 * jj;
                    kr[b][p].load(k + off);
                    qr[b][p].load(q + off);
                } else {
                    kr[b][p].zero();
                    qr[b][p].zero();
                }
            }
        }
    };
    load(0);
    float la = 0.f, bt = 0.f;
    if (l < len) {
        const int64_t th = (int64_t)(tok0 + l) * H + h;
        la = log_alpha[th];
        bt = beta[th];
    }
    const float g = wave_inclusive_scan(la);
    const float glast = __shfl(g, C - 1, 64);
    sg[l] = g;
    sb[l] = bt;
    float *vec = ws_vec + (int64_t)item * kVecFloats;
    vec[l] = g;
    vec[C + l] = expf(g);
    vec[2 * C + l] = expf(glast - g);
    vec[3 * C + l] = bt;

    // Lower tiles t = (a, b) of K K^T and Q K^T, R layout.
    float4_t kk[kTriTiles], qk[kTriTiles];
#pragma unroll
    for (int t = 0; t < kTriTiles; ++t) kk[t] = qk[t] = zero4();
#pragma unroll
    for (int s = 0; s < NPASS; ++s) {
        if (s > 0) load(s);
#pragma unroll
        for (int t = 0; t < kTriTiles; ++t) {
            int a, b;
            tri_decode(t, a, b);
#pragma unroll
            for (int p = 0; p < PP; ++p) {
                gram_mma(kk[t], kr[b][p], kr[a][p]);
                gram_mma(qk[t], kr[b][p], qr[a][p]);
            }
        }
    }

    // Decay masks.  P = (Q K^T) o Gamma and G = (K K^T) o Gamma (lower with the
    // diagonal) to HBM; -A for the off-diagonal tiles in registers, N_a^T of
    // the diagonal blocks to LDS (blk[a][c][m] = A[16a + m][16a + c], m > c).
    float *P = ws_p + (int64_t)item * C * C, *G = ws_g + (int64_t)item * C * C, *Tm = ws_t + (int64_t)item * C * C;
    float gr[4], br[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        gr[a] = sg[16 * a + nn];
        br[a] = sb[16 * a + nn];
    }
    float4_t naR[kTriTiles];   // R(-A_ab), a > b
#pragma unroll
    for (int t = 0; t < kTriTiles; ++t) {
        int a, b;
        tri_decode(t, a, b);
        const float4_t gc = *reinterpret_cast<const float4_t *>(sg + 16 * b + 4 * jj);
        float4_t pv, gv, av;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * a + nn, c = 16 * b + 4 * jj + i;
            const float gm = c <= r ? expf(gr[a] - gc[i]) : 0.f;
            pv[i] = qk[t][i] * gm;
            gv[i] = kk[t][i] * gm;
            av[i] = c < r ? br[a] * gm * kk[t][i] : 0.f;
        }
        const int64_t o = (int64_t)(16 * a + nn) * C + 16 * b + 4 * jj;
        *reinterpret_cast<float4_t *>(P + o) = pv;
        *reinterpret_cast<float4_t *>(G + o) = gv;
        if (a > b) {
            naR[t] = -av;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) blk[a * BS + (4 * jj + i) * BP + nn] = av[i];
            naR[t] = zero4();
        }
    }
    // the upper tiles of P, G and T are zero
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = a + 1; b < 4; ++b) {
            const int64_t o = (int64_t)(16 * a + nn) * C + 16 * b + 4 * jj;
            *reinterpret_cast<float4_t *>(P + o) = zero4();
            *reinterpret_cast<float4_t *>(G + o) = zero4();
            *reinterpret_cast<float4_t *>(Tm + o) = zero4();
        }
    asm volatile("" ::: "memory");   // one wave: only the compiler could reorder its LDS accesses
    // Diagonal blocks: lane (n, j) solves row n of T_jj.
    diag_block_inverse<BP, BS>(blk, nn, jj);
    float4_t tR[4], tC[3];   // R(T_aa), C(T_bb)
#pragma unroll
    for (int a = 0; a < 4; ++a) tR[a] = *reinterpret_cast<const float4_t *>(blk + a * BS + nn * BP + 4 * jj);
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) tC[b][i] = blk[b * BS + (4 * jj + i) * BP + nn];

    // Off-diagonal blocks by distance; C layouts where a later W needs them.
    const float4_t z = zero4();
    float4_t W, T10, T21, T32, T20, T31, T30, C10, C21, C20;
    W = mm16_f32(naR[tri_index(1, 0)], tC[0], z);
    T10 = mm16_f32(W, tR[1], z);
    C10 = mm16_f32(tR[1], W, z);
    W = mm16_f32(naR[tri_index(2, 1)], tC[1], z);
    T21 = mm16_f32(W, tR[2], z);
    C21 = mm16_f32(tR[2], W, z);
    W = mm16_f32(naR[tri_index(3, 2)], tC[2], z);
    T32 = mm16_f32(W, tR[3], z);
    W = mm16_f32(naR[tri_index(2, 1)], C10, mm16_f32(naR[tri_index(2, 0)], tC[0], z));
    T20 = mm16_f32(W, tR[2], z);
    C20 = mm16_f32(tR[2], W, z);
    W = mm16_f32(naR[tri_index(3, 2)], C21, mm16_f32(naR[tri_index(3, 1)], tC[1], z));
    T31 = mm16_f32(W, tR[3], z);
    W = mm16_f32(naR[tri_index(3, 2)], C20, mm16_f32(naR[tri_index(3, 1)], C10, mm16_f32(naR[tri_index(3, 0)], tC[0], z)));
    T30 = mm16_f32(W, tR[3], z);

    auto put = [&](int a, int b, const float4_t &x) {
        *reinterpret_cast<float4_t *>(Tm + (int64_t)(16 * a + nn) * C + 16 * b + 4 * jj) = x;
    };
    put(0, 0, tR[0]);
    put(1, 0, T10);
    put(1, 1, tR[1]);
    put(2, 0, T20);
    put(2, 1, T21);
    put(2, 2, tR[2]);
    put(3, 0, T30);
    put(3, 1, T31);
    put(3, 2, T32);
    put(3, 3, tR[3]);
}

// ============================================================================
// B2: the state pass again, storing the state at every chunk start.
// One 256-thread block per (sequence, head, 16 value columns).  S^T for the
// columns (dk x 16) lives in DK / 16 accumulator tiles spread over the four
// waves (wave w holds tiles w, w + 4, ...): tile a, element i of lane (n, j)
// = S[v0 + n][16 a + 4 j + i].  Per chunk wave w forms rows 16 w .. 16 w + 15
// of X = K S^T, Y and V' = M Y; the tiles, Y and V' pass through LDS.
// ============================================================================
// Position of element (x, r) of a transposed C x C matrix (row x) in LDS:
// the row's 4-float groups are XOR-permuted by a function of x, so the
// staging writes (16 lanes, x = 4 t + i, one r) fall in distinct banks
// while a lane's four consecutive r of one row stay one 16-byte read.
__device__ __forceinline__ int tswz(int x, int r) { return x * (C + 4) + (r ^ (4 * ((x >> 2) & 15))); }

// bf16 form of the state-pass products for bf16 inputs.  K's values are bf16,
// and an fp32 value is the exact sum of three bf16 values: its upper 8
// significant bits, the next 8 (the remainder after the first cut is exact in
// fp32) and the last 8.  A product with K then takes three bf16 matrix-core
// instructions (products exact, sums fp32) for each 32-wide k slice instead of
// eight fp32 ones, at the precision of the fp32 product.
template <typename T>
struct SplitState {
    static constexpr bool value = false;
};
template <>
struct SplitState<bf16_t> {
    static constexpr bool value = true;
};
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// acc += A B over one 32-wide k slice: lane (n, j) supplies A[n][8j .. 8j + 7]
// and B[8j .. 8j + 7][n] as four packed bf16 pairs each.
__device__ __forceinline__ void mfma_bf16(float4_t &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), acc,
                                                 0, 0, 0);
}
// The upper halves of two fp32 words as one bf16 pair, x0 first (exact when
// both values are bf16 values).
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
    return __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
}
// x = hi + mid + lo exactly, each a bf16 value, as packed pairs.
__device__ __forceinline__ void split3(const float4_t &x, uint2 &hi, uint2 &mid, uint2 &lo) {
    float h[4], m[4], r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = __uint_as_float(__float_as_uint(x[e]) & 0xffff0000u);
        const float r1 = x[e] - h[e];
        m[e] = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
        r[e] = r1 - m[e];
    }
    hi = uint2{pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3])};
    mid = uint2{pack_bf16(m[0], m[1]), pack_bf16(m[2], m[3])};
    lo = uint2{pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3])};
}

template <int DK, bool SPL>
struct PassSmem {
    static constexpr int KP = DK + 4;   // rows of K; rows of the state tile (S, 16 x DK)
    static constexpr int TP = C + 4;    // transposed value blocks [16][C]; C x C matrices
    static constexpr int SBP = DK + 8;  // split form: bf16 rows of K and of the three state terms
    static constexpr int VBP = C + 8;   // split form: bf16 rows of the three (diag(kappa) V')^T terms
    static constexpr int off_k = 0;                                       // K rows (bf16 in split form)
    static constexpr int off_s = off_k + (SPL ? C * SBP / 2 : C * KP);    // S rows (or their three bf16 terms)
    static constexpr int off_a = off_s + (SPL ? 3 * 16 * SBP / 2 : 16 * KP);  // Y^T
    static constexpr int off_b = off_a + 16 * TP;                         // (diag(kappa) V')^T (or its terms)
    static constexpr int off_m = off_b + (SPL ? 3 * 16 * VBP / 2 : 16 * TP);  // M = T diag(beta)
    static constexpr int off_v = off_m + C * TP;                          // gamma, kappa, beta
    static constexpr size_t bytes_fwd = sizeof(float) * (off_v + 3 * C);
};

// LDS of the reverse pass (two 16-column tiles per block): shared K rows,
// (diag(gamma) Q)^T, T^T and P^T (all three swizzled, tswz), the decay
// vectors; per tile the dS rows and the transposed dO, dV', -diag(gamma) dY
// blocks.
// In the split form (bf16 inputs, see SplitState) K and Q are bf16 rows, and
// the dS rows, -diag(gamma) dY and an extra (diag(gamma) dO)^T hold three bf16
// terms each.
template <int DK, bool SPL>
struct RevSmem {
    static constexpr int KP = DK + 4, TP = C + 4;
    static constexpr int KB = DK + 8;   // split form: bf16 rows of K, Q and of the dS terms
    static constexpr int VB = C + 8;    // split form: bf16 rows of the transposed value-side terms
    static constexpr int off_k = 0;                                       // K rows
    static constexpr int off_q = off_k + (SPL ? C * KB / 2 : C * KP);    // Q rows, or (diag(gamma) Q)^T
    static constexpr int off_m = off_q + (SPL ? C * KB / 2 : DK * TP);   // T^T
    static constexpr int off_p = off_m + C * TP;       // P^T
    static constexpr int off_v = off_p + C * TP;       // gamma, kappa, beta
    static constexpr int off_t0 = off_v + 3 * C;       // per-tile blocks:
    static constexpr int S_FL = SPL ? 3 * 16 * KB / 2 : 16 * KP;   //   dS rows
    static constexpr int Y_FL = SPL ? 3 * 16 * VB / 2 : 16 * TP;   //   (-diag(gamma) dY)^T
    static constexpr int G_FL = SPL ? 3 * 16 * VB / 2 : 0;         //   (diag(gamma) dO)^T
    static constexpr int t_s = 0, t_o = S_FL, t_dvp = t_o + 16 * TP, t_dy = t_dvp + 16 * TP, t_og = t_dy + Y_FL;
    static constexpr int TILE = t_og + G_FL;           //   (with dO^T and dV'^T)
    static constexpr size_t bytes = sizeof(float) * (off_t0 + 2 * TILE);
    static_assert(bytes <= 160 * 1024, "reverse pass fits the 160 KiB of LDS");
    static_assert(off_t0 % 4 == 0 && TILE % 4 == 0, "16-byte aligned blocks");
};

// One chunk's operands of the forward pass, loaded into registers while the
// previous chunk computes (thread tid covers K elements tid * 8 + 2048 m,
// T elements tid * 4 + 1024 m, the V values of its lane's accumulator rows,
// and vector element tid).  Every load is unconditional (rows past the
// chunk's end re-read its last row and are zeroed on use), so no wait is
// attached to a load right after it is issued.
template <typename in_t, int DK>
struct PassStage {
    static constexpr int MK = C * DK / 2048;
    int tok0, len;
    int64_t item;
    Raw8<in_t> kr[MK];
    float4_t t4[4], b4;
    in_t vv[4];
    float vec;
};

template <typename in_t, int DK>
__device__ __forceinline__ void pass_load(PassStage<in_t, DK> &S, int row, int H, int h, int DV, int v0, int T,
                                          int cpr, const int32_t *row_tok, const int32_t *row_len, const in_t *k,
                                          const in_t *v, const float *ws_t, const float *ws_vec) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, nn = l & 15, jj = l >> 4;
    row_span(row, T, cpr, row_tok, row_len, S.tok0, S.len);
    S.item = (int64_t)row * H + h;
#pragma unroll
    for (int m = 0; m < PassStage<in_t, DK>::MK; ++m) {
        const int idx = tid * 8 + 2048 * m, r = min(idx / DK, S.len - 1), cc = idx % DK;
        S.kr[m].load(k + ((int64_t)(S.tok0 + r) * H + h) * DK + cc);
    }
    const float *Tm = ws_t + S.item * C * C, *vec = ws_vec + S.item * kVecFloats;
#pragma unroll
    for (int m = 0; m < 4; ++m) S.t4[m] = *reinterpret_cast<const float4_t *>(Tm + tid * 4 + 1024 * m);
    S.b4 = *reinterpret_cast<const float4_t *>(vec + 3 * C + (tid * 4) % C);
    S.vec = vec[C + min(tid, 3 * C - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = min(16 * w + 4 * jj + i, S.len - 1);
        S.vv[i] = v[((int64_t)(S.tok0 + r) * H + h) * DV + v0 + nn];
    }
}

// Writes a staged chunk into LDS (layout of PassSmem): K rows, M = T diag(beta),
// gamma, kappa, beta.
template <typename in_t, int DK>
__device__ __forceinline__ void pass_store(const PassStage<in_t, DK> &S, float *smem) {
    constexpr bool SPL = SplitState<in_t>::value;
    using L = PassSmem<DK, SPL>;
    constexpr int KP = L::KP, TP = L::TP, SBP = L::SBP;
    float *sk = smem + L::off_k, *sm = smem + L::off_m, *sv = smem + L::off_v;
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < PassStage<in_t, DK>::MK; ++m) {
        const int idx = tid * 8 + 2048 * m, r = idx / DK, cc = idx % DK;
        if constexpr (SPL) {   // bf16 rows as they are
            Raw8<in_t> kk = S.kr[m];
            if (r >= S.len) kk.zero();
            kk.store_lds(reinterpret_cast<in_t *>(sk) + r * SBP + cc);
            continue;
        }
        float x[8];
        S.kr[m].to_f32(x);
        if (r >= S.len)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
        *reinterpret_cast<float4_t *>(sk + r * KP + cc) = float4_t{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<float4_t *>(sk + r * KP + cc + 4) = float4_t{x[4], x[5], x[6], x[7]};
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = tid * 4 + 1024 * m, r = e / C, cc = e % C;
        *reinterpret_cast<float4_t *>(sm + r * TP + cc) = S.t4[m] * S.b4;
    }
    if (tid < 3 * C) sv[tid] = S.vec;
}

template <typename in_t, int DK>
__global__ __launch_bounds__(256) void bwd_fwd_pass_kernel(int NH, int H, int DV, int T, int cpr, int nvt,
                                                           const int32_t *__restrict__ meta,
                                                           const int32_t *__restrict__ cu_ws,
                                                           const int32_t *__restrict__ row0,
                                                           const int32_t *__restrict__ row_tok,
                                                           const int32_t *__restrict__ row_len,
                                                           const in_t *__restrict__ k, const in_t *__restrict__ v,
                                                           const float *__restrict__ ws_t,
                                                           const float *__restrict__ ws_vec,
                                                           const float *__restrict__ init_state,
                                                           float *__restrict__ ws_ck, float *__restrict__ ws_y,
                                                           float *__restrict__ ws_vp) {
    constexpr bool SPL = SplitState<in_t>::value;
    using L = PassSmem<DK, SPL>;
    constexpr int KP = L::KP, TP = L::TP, SBP = L::SBP, VBP = L::VBP, NA = DK / 16, NT = (NA + 3) / 4;
    extern __shared__ __align__(16) float smem[];
    float *sk = smem + L::off_k, *ss = smem + L::off_s, *syt = smem + L::off_a, *svpt = smem + L::off_b;
    float *sm = smem + L::off_m, *sv = smem + L::off_v;   // sv: gamma [C], kappa [C], beta [C]
    uint16_t *ssb = reinterpret_cast<uint16_t *>(ss), *svb = reinterpret_cast<uint16_t *>(svpt);   // split form
    const uint16_t *skb = reinterpret_cast<const uint16_t *>(sk);                                   // split form: K rows
    if (!cpr && meta[1] != 0) return;
    // The value tiles of one (sequence, head) read the same K and T.  Blocks
    // are dealt to the 8 XCDs in turn, so give a head's tiles block indices
    // equal mod 8: they then share one XCD's L2.
    const int bid = blockIdx.x, slot = bid >> 3;
    const int nh = (slot / nvt) * 8 + (bid & 7), vt = slot % nvt;
    if (nh >= NH) return;
    const int n = nh / H, h = nh % H, v0 = vt * 16;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, nn = l & 15, jj = l >> 4;
    int r0, nrows;
    seq_rows(n, T, cpr, cu_ws, row0, r0, nrows);

    float4_t s[NT];   // tiles a = w + 4 t
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int a = w + 4 * t;
        s[t] = (init_state && a < NA)
                   ? *reinterpret_cast<const float4_t *>(init_state + ((int64_t)nh * DV + v0 + nn) * DK + 16 * a + 4 * jj)
                   : zero4();
    }
    PassStage<in_t, DK> S;
    if (nrows > 0) pass_load(S, r0, H, h, DV, v0, T, cpr, row_tok, row_len, k, v, ws_t, ws_vec);
    const int rw = 16 * w;
    // Y and V' of the previous chunk, stored once the next chunk's operands
    // have landed: a wave's loads and stores share one completion counter that
    // need not drain in order, so a wait for loads also waits for every store
    // issued before it.  Stores therefore go out right after a wait and
    // before the next loads, a whole chunk ahead of the next wait.
    float4_t py = zero4(), pvp = zero4();
    int64_t pitem = -1;
    auto store_yv = [&]() {
        if (pitem >= 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t o = pitem * C * DV + (int64_t)v0 * C + (rw + 4 * jj + i) * 16 + nn;   // block-major
                ws_y[o] = py[i];
                ws_vp[o] = pvp[i];
            }
        }
    };
    for (int c = 0; c < nrows; ++c) {
        const int len = S.len;
        const int64_t item = S.item;
        float vv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = 16 * w + 4 * jj + i < len ? to_f32(S.vv[i]) : 0.f;
        __syncthreads();   // the previous chunk's LDS contents are no longer read
        pass_store(S, smem);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int a = w + 4 * t;
            if (a < NA) {
                if constexpr (SPL) {   // row v0 + n of S as three bf16 terms
                    uint2 hi, mid, lo;
                    split3(s[t], hi, mid, lo);
                    const int o = nn * SBP + 16 * a + 4 * jj;
                    *reinterpret_cast<uint2 *>(ssb + o) = hi;
                    *reinterpret_cast<uint2 *>(ssb + 16 * SBP + o) = mid;
                    *reinterpret_cast<uint2 *>(ssb + 32 * SBP + o) = lo;
                } else {
                    *reinterpret_cast<float4_t *>(ss + nn * KP + 16 * a + 4 * jj) = s[t];   // row v0 + n of S
                }
                *reinterpret_cast<float4_t *>(ws_ck + (item * DV + v0 + nn) * DK + 16 * a + 4 * jj) = s[t];
            }
        }
        store_yv();
        // the next chunk's operands load while this one computes (the last
        // chunk loads itself again)
        pass_load(S, r0 + min(c + 1, nrows - 1), H, h, DV, v0, T, cpr, row_tok, row_len, k, v, ws_t, ws_vec);
        __syncthreads();
        const float glast = len > 0 ? sv[len - 1] : 1.f;
        // rows of the wave: X = K S^T, Y = V - diag(gamma) X
        float4_t x = zero4();
        if constexpr (SPL) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const uint4 ka = *reinterpret_cast<const uint4 *>(skb + (rw + nn) * SBP + 32 * ks + 8 * jj);
#pragma unroll
                for (int term = 0; term < 3; ++term)
                    mfma_bf16(x, ka, *reinterpret_cast<const uint4 *>(ssb + (16 * term + nn) * SBP + 32 * ks + 8 * jj));
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < NA; ++kt) {
                const float4_t a4 = *reinterpret_cast<const float4_t *>(sk + (rw + nn) * KP + 16 * kt + 4 * jj);
                const float4_t b4 = *reinterpret_cast<const float4_t *>(ss + nn * KP + 16 * kt + 4 * jj);
#pragma unroll
                for (int i = 0; i < 4; ++i) mfma4(x, a4[i], b4[i]);
            }
        }
        float4_t y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = vv[i] - sv[rw + 4 * jj + i] * x[i];
        *reinterpret_cast<float4_t *>(syt + nn * TP + rw + 4 * jj) = y;
        __syncthreads();
        // V' = M Y, M lower block triangular
        float4_t vp = zero4();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            if (kt <= w) {
                const float4_t a4 = *reinterpret_cast<const float4_t *>(sm + (rw + nn) * TP + 16 * kt + 4 * jj);
                const float4_t b4 = *reinterpret_cast<const float4_t *>(syt + nn * TP + 16 * kt + 4 * jj);
#pragma unroll
                for (int i = 0; i < 4; ++i) mfma4(vp, a4[i], b4[i]);
            }
        }
        py = y;
        pvp = vp;
        pitem = item;
        float4_t kvp;   // diag(kappa) V', the operand of the state update
#pragma unroll
        for (int i = 0; i < 4; ++i) kvp[i] = sv[C + rw + 4 * jj + i] * vp[i];
        if constexpr (SPL) {
            uint2 hi, mid, lo;
            split3(kvp, hi, mid, lo);
            const int o = nn * VBP + rw + 4 * jj;
            *reinterpret_cast<uint2 *>(svb + o) = hi;
            *reinterpret_cast<uint2 *>(svb + 16 * VBP + o) = mid;
            *reinterpret_cast<uint2 *>(svb + 32 * VBP + o) = lo;
        } else {
            *reinterpret_cast<float4_t *>(svpt + nn * TP + rw + 4 * jj) = kvp;
        }
        __syncthreads();
        // S^T <- gamma_last S^T + K^T (diag(kappa) V') on the wave's tiles
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int a = w + 4 * t;
            if (a < NA) {
                float4_t acc = glast * s[t];
                if constexpr (SPL) {
#pragma unroll
                    for (int ks = 0; ks < C / 32; ++ks) {
                        const uint4 ka = lds_col8_b16(skb, SBP, 32 * ks, 16 * a, nn, jj);   // K^T fragment
#pragma unroll
                        for (int term = 0; term < 3; ++term)
                            mfma_bf16(acc, ka,
                                      *reinterpret_cast<const uint4 *>(svb + (16 * term + nn) * VBP + 32 * ks + 8 * jj));
                    }
                } else {
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) {
                        const float4_t b4 = *reinterpret_cast<const float4_t *>(svpt + nn * TP + 16 * kt + 4 * jj);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int kx = 16 * kt + 4 * jj + i;
                            mfma4(acc, sk[kx * KP + 16 * a + nn], b4[i]);
                        }
                    }
                }
                s[t] = acc;
            }
        }
    }
    store_yv();
}

// ============================================================================
// B3: the reverse state pass.  One 8-wave block per (sequence, head, pair of
// 16-column value tiles): waves 4 p .. 4 p + 3 carry tile p's dS^T in the
// layout of B2 (wave w & 3 holds tiles (w & 3) + 4 t and computes chunk rows
// 16 (w & 3) ..), and the two tiles share the staged K, Q, T and P.  Chunks
// in reverse: store dS (the gradient of the state at the chunk's end), then
//   dV' = P^T dO + diag(kappa) K dS^T,  dY = M^T dV' = diag(beta) T^T dV',
//   dS  <- gamma_last dS + dO^T diag(gamma) Q - dY^T diag(gamma) K.
// What is left after the first chunk is the initial state's gradient.
// ============================================================================
template <typename in_t, int DK>
struct RevStage {
    static constexpr int MK = (C * DK + 4095) / 4096;   // K / Q elements tid * 8 + 4096 m
    int tok0, len;
    int64_t item;
    Raw8<in_t> kr[MK], qr[MK];
    float gq[MK];            // gamma of the row of K / Q group m
    float gdo[4];            // gamma of the row of dO element m
    float4_t t4[2], p4[2];   // T / P elements tid * 4 + 2048 m
    float dov[4];            // dO element tid + 512 m of the two tiles' value blocks
    float vec;
};

template <typename in_t, int DK>
__device__ __forceinline__ void rev_load(RevStage<in_t, DK> &S, int row, int H, int h, int DV, int vpair, int nvt,
                                         int T, int cpr, const int32_t *row_tok, const int32_t *row_len,
                                         const in_t *q, const in_t *k, const float *d_o, const float *ws_t,
                                         const float *ws_p, const float *ws_vec) {
    const int tid = threadIdx.x;
    row_span(row, T, cpr, row_tok, row_len, S.tok0, S.len);
    S.item = (int64_t)row * H + h;
    const float *Tm = ws_t + S.item * C * C, *Pm = ws_p + S.item * C * C, *vec = ws_vec + S.item * kVecFloats;
#pragma unroll
    for (int m = 0; m < RevStage<in_t, DK>::MK; ++m) {
        const int idx = tid * 8 + 4096 * m, r = idx / DK, cc = idx % DK;
        const int64_t off = ((int64_t)(S.tok0 + r) * H + h) * DK + cc;
        if (idx < C * DK && r < S.len) {
            S.kr[m].load(k + off);
            S.qr[m].load(q + off);
            S.gq[m] = vec[C + r];
        } else {
            S.kr[m].zero();
            S.qr[m].zero();
            S.gq[m] = 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        S.t4[m] = *reinterpret_cast<const float4_t *>(Tm + tid * 4 + 2048 * m);
        S.p4[m] = *reinterpret_cast<const float4_t *>(Pm + tid * 4 + 2048 * m);
    }
    S.vec = tid < 3 * C ? vec[C + tid] : 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = tid + 512 * m, tile = e / 1024, r = (e % 1024) / 16, cc = e % 16;
        const int vt = 2 * vpair + tile;
        S.dov[m] = (vt < nvt && r < S.len) ? d_o[((int64_t)(S.tok0 + r) * H + h) * DV + 16 * vt + cc] : 0.f;
        if constexpr (SplitState<in_t>::value) S.gdo[m] = r < S.len ? vec[C + r] : 0.f;
    }
}

template <typename in_t, int DK>
__device__ __forceinline__ void rev_store(const RevStage<in_t, DK> &S, float *smem) {
    constexpr bool SPL = SplitState<in_t>::value;
    using L = RevSmem<DK, SPL>;
    constexpr int KP = L::KP, TP = L::TP, KB = L::KB, VB = L::VB;
    float *sk = smem + L::off_k, *sqt = smem + L::off_q, *sm = smem + L::off_m, *sp = smem + L::off_p;
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < RevStage<in_t, DK>::MK; ++m) {
        const int idx = tid * 8 + 4096 * m, r = idx / DK, cc = idx % DK;
        if (SPL && idx < C * DK) {   // K and Q rows as they are (bf16)
            S.kr[m].store_lds(reinterpret_cast<in_t *>(sk) + r * KB + cc);
            S.qr[m].store_lds(reinterpret_cast<in_t *>(sqt) + r * KB + cc);
        } else if (idx < C * DK) {
            float x[8];
            S.kr[m].to_f32(x);
            *reinterpret_cast<float4_t *>(sk + r * KP + cc) = float4_t{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<float4_t *>(sk + r * KP + cc + 4) = float4_t{x[4], x[5], x[6], x[7]};
            S.qr[m].to_f32(x);
#pragma unroll
            for (int e = 0; e < 8; ++e) sqt[tswz(cc + e, r)] = S.gq[m] * x[e];   // (diag(gamma) Q)^T
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int e = tid * 4 + 2048 * m, r = e / C, cc = e % C;
#pragma unroll
        for (int i = 0; i < 4; ++i) {   // T^T (diag(beta) is applied to T^T dV') and P^T, swizzled
            sm[tswz(cc + i, r)] = S.t4[m][i];
            sp[tswz(cc + i, r)] = S.p4[m][i];
        }
    }
    if (tid < 3 * C) smem[L::off_v + tid] = S.vec;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = tid + 512 * m, tile = e / 1024, r = (e % 1024) / 16, cc = e % 16;
        smem[L::off_t0 + tile * L::TILE + L::t_o + cc * TP + r] = S.dov[m];
        if constexpr (SPL) {   // (diag(gamma) dO)^T as three bf16 terms
            uint16_t *og = reinterpret_cast<uint16_t *>(smem + L::off_t0 + tile * L::TILE + L::t_og) + cc * VB + r;
            const float g = S.gdo[m] * S.dov[m];
            const float hi = __uint_as_float(__float_as_uint(g) & 0xffff0000u), r1 = g - hi;
            const float mid = __uint_as_float(__float_as_uint(r1) & 0xffff0000u), lo = r1 - mid;
            og[0] = (uint16_t)(__float_as_uint(hi) >> 16);
            og[16 * VB] = (uint16_t)(__float_as_uint(mid) >> 16);
            og[32 * VB] = (uint16_t)(__float_as_uint(lo) >> 16);
        }
    }
}

template <typename in_t, int DK>
__global__ __launch_bounds__(512) void bwd_rev_pass_kernel(int NH, int H, int DV, int T, int cpr, int nvt,
                                                           const int32_t *__restrict__ meta,
                                                           const int32_t *__restrict__ cu_ws,
                                                           const int32_t *__restrict__ row0,
                                                           const int32_t *__restrict__ row_tok,
                                                           const int32_t *__restrict__ row_len,
                                                           const in_t *__restrict__ q, const in_t *__restrict__ k,
                                                           const float *__restrict__ d_o,
                                                           const float *__restrict__ ws_t,
                                                           const float *__restrict__ ws_p,
                                                           const float *__restrict__ ws_vec,
                                                           const float *__restrict__ d_final,
                                                           float *__restrict__ ws_ds, float *__restrict__ ws_dvp,
                                                           float *__restrict__ dv, float *__restrict__ d_init) {
    constexpr bool SPL = SplitState<in_t>::value;
    using L = RevSmem<DK, SPL>;
    constexpr int KP = L::KP, TP = L::TP, KB = L::KB, VB = L::VB, NA = DK / 16, NT = (NA + 3) / 4;
    extern __shared__ __align__(16) float smem[];
    if (!cpr && meta[1] != 0) return;
    const int npair = (nvt + 1) / 2;
    const int bid = blockIdx.x, slot = bid >> 3;   // a head's tile pairs on one XCD, as in the forward pass
    const int nh = (slot / npair) * 8 + (bid & 7), vpair = slot % npair;
    if (nh >= NH) return;
    const int n = nh / H, h = nh % H;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, nn = l & 15, jj = l >> 4;
    const int tile = w >> 2, wr = w & 3, vt = 2 * vpair + tile, v0 = 16 * vt;
    const bool active = vt < nvt;
    const float *sk = smem + L::off_k, *sqt = smem + L::off_q, *smt = smem + L::off_m, *spt = smem + L::off_p;
    const float *sv = smem + L::off_v;
    float *tb = smem + L::off_t0 + tile * L::TILE;
    float *ss = tb + L::t_s, *sot = tb + L::t_o, *sdvpt = tb + L::t_dvp, *sdyt = tb + L::t_dy;
    // split form: bf16 K and Q rows, the terms of dS, of -diag(gamma) dY and of diag(gamma) dO
    const uint16_t *skb = reinterpret_cast<const uint16_t *>(sk), *sqb = reinterpret_cast<const uint16_t *>(sqt);
    uint16_t *ssb = reinterpret_cast<uint16_t *>(ss), *syb = reinterpret_cast<uint16_t *>(sdyt);
    const uint16_t *sgb = reinterpret_cast<const uint16_t *>(tb + L::t_og);
    int r0, nrows;
    seq_rows(n, T, cpr, cu_ws, row0, r0, nrows);

    float4_t s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int a = wr + 4 * t;
        s[t] = (active && d_final && a < NA)
                   ? *reinterpret_cast<const float4_t *>(d_final + ((int64_t)nh * DV + v0 + nn) * DK + 16 * a + 4 * jj)
                   : zero4();
    }
    RevStage<in_t, DK> S;
    if (nrows > 0)
        rev_load(S, r0 + nrows - 1, H, h, DV, vpair, nvt, T, cpr, row_tok, row_len, q, k, d_o, ws_t, ws_p, ws_vec);
    const int rw = 16 * wr;
    for (int c = nrows - 1; c >= 0; --c) {
        const int tok0 = S.tok0, len = S.len;
        const int64_t item = S.item;
        __syncthreads();
        if (active) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int a = wr + 4 * t;
                if (a < NA) {
                    *reinterpret_cast<float4_t *>(ws_ds + (item * DV + v0 + nn) * DK + 16 * a + 4 * jj) = s[t];
                    if constexpr (SPL) {   // row v0 + n of dS as three bf16 terms
                        uint2 hi, mid, lo;
                        split3(s[t], hi, mid, lo);
                        const int o = nn * KB + 16 * a + 4 * jj;
                        *reinterpret_cast<uint2 *>(ssb + o) = hi;
                        *reinterpret_cast<uint2 *>(ssb + 16 * KB + o) = mid;
                        *reinterpret_cast<uint2 *>(ssb + 32 * KB + o) = lo;
                    } else {
                        *reinterpret_cast<float4_t *>(ss + nn * KP + 16 * a + 4 * jj) = s[t];   // row v0 + n of dS
                    }
                }
            }
        }
        rev_store(S, smem);
        if (c > 0)   // the next chunk's operands load while this one computes
            rev_load(S, r0 + c - 1, H, h, DV, vpair, nvt, T, cpr, row_tok, row_len, q, k, d_o, ws_t, ws_p, ws_vec);
        __syncthreads();
        const float glast = len > 0 ? sv[len - 1] : 1.f;
        // dV' = P^T dO + diag(kappa) K dS^T on the wave's rows
        if (active) {
            float4_t x = zero4();
            if constexpr (SPL) {
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const uint4 ka = *reinterpret_cast<const uint4 *>(skb + (rw + nn) * KB + 32 * ks + 8 * jj);
#pragma unroll
                    for (int term = 0; term < 3; ++term)
                        mfma_bf16(x, ka, *reinterpret_cast<const uint4 *>(ssb + (16 * term + nn) * KB + 32 * ks + 8 * jj));
                }
            } else {
#pragma unroll
                for (int kt = 0; kt < NA; ++kt) {
                    const float4_t a4 = *reinterpret_cast<const float4_t *>(sk + (rw + nn) * KP + 16 * kt + 4 * jj);
                    const float4_t b4 = *reinterpret_cast<const float4_t *>(ss + nn * KP + 16 * kt + 4 * jj);
#pragma unroll
                    for (int i = 0; i < 4; ++i) mfma4(x, a4[i], b4[i]);
                }
            }
            float4_t dvp;
#pragma unroll
            for (int i = 0; i < 4; ++i) dvp[i] = sv[C + rw + 4 * jj + i] * x[i];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (kt >= wr) {
                    const float4_t a4 = *reinterpret_cast<const float4_t *>(spt + tswz(rw + nn, 16 * kt + 4 * jj));
                    const float4_t b4 = *reinterpret_cast<const float4_t *>(sot + nn * TP + 16 * kt + 4 * jj);
#pragma unroll
                    for (int i = 0; i < 4; ++i) mfma4(dvp, a4[i], b4[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) ws_dvp[(int64_t)item * C * DV + (int64_t)v0 * C + (rw + 4 * jj + i) * 16 + nn] = dvp[i];
            *reinterpret_cast<float4_t *>(sdvpt + nn * TP + rw + 4 * jj) = dvp;
        }
        __syncthreads();
        // dY = M^T dV' = diag(beta) T^T dV'
        if (active) {
            float4_t dy = zero4();
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (kt >= wr) {
                    const float4_t a4 = *reinterpret_cast<const float4_t *>(smt + tswz(rw + nn, 16 * kt + 4 * jj));
                    const float4_t b4 = *reinterpret_cast<const float4_t *>(sdvpt + nn * TP + 16 * kt + 4 * jj);
#pragma unroll
                    for (int i = 0; i < 4; ++i) mfma4(dy, a4[i], b4[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rw + 4 * jj + i;
                dy[i] *= sv[2 * C + r];
                if (r < len) dv[((int64_t)(tok0 + r) * H + h) * DV + v0 + nn] = dy[i];
            }
            float4_t ndy;   // -diag(gamma) dY, the operand of the state update
#pragma unroll
            for (int i = 0; i < 4; ++i) ndy[i] = -sv[rw + 4 * jj + i] * dy[i];
            if constexpr (SPL) {
                uint2 hi, mid, lo;
                split3(ndy, hi, mid, lo);
                const int o = nn * VB + rw + 4 * jj;
                *reinterpret_cast<uint2 *>(syb + o) = hi;
                *reinterpret_cast<uint2 *>(syb + 16 * VB + o) = mid;
                *reinterpret_cast<uint2 *>(syb + 32 * VB + o) = lo;
            } else {
                *reinterpret_cast<float4_t *>(sdyt + nn * TP + rw + 4 * jj) = ndy;
            }
        }
        __syncthreads();
        // dS^T <- gamma_last dS^T + (diag(gamma) Q)^T dO + K^T (-diag(gamma) dY) on the wave's tiles
        if (active) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int a = wr + 4 * t;
                if (a < NA) {
                    float4_t acc = glast * s[t];
                    if constexpr (SPL) {   // Q^T (diag(gamma) dO) + K^T (-diag(gamma) dY)
#pragma unroll
                        for (int ks = 0; ks < C / 32; ++ks) {
                            const uint4 qa = lds_col8_b16(sqb, KB, 32 * ks, 16 * a, nn, jj);   // Q^T fragment
                            const uint4 ka = lds_col8_b16(skb, KB, 32 * ks, 16 * a, nn, jj);   // K^T fragment
#pragma unroll
                            for (int term = 0; term < 3; ++term) {
                                const int o = (16 * term + nn) * VB + 32 * ks + 8 * jj;
                                mfma_bf16(acc, qa, *reinterpret_cast<const uint4 *>(sgb + o));
                                mfma_bf16(acc, ka, *reinterpret_cast<const uint4 *>(syb + o));
                            }
                        }
                    } else {
#pragma unroll
                        for (int kt = 0; kt < 4; ++kt) {
                            const float4_t bo = *reinterpret_cast<const float4_t *>(sot + nn * TP + 16 * kt + 4 * jj);
                            const float4_t by = *reinterpret_cast<const float4_t *>(sdyt + nn * TP + 16 * kt + 4 * jj);
                            const float4_t aq = *reinterpret_cast<const float4_t *>(sqt + tswz(16 * a + nn, 16 * kt + 4 * jj));
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int kx = 16 * kt + 4 * jj + i;
                                mfma4(acc, aq[i], bo[i]);
                                mfma4(acc, sk[kx * KP + 16 * a + nn], by[i]);
                            }
                        }
                    }
                    s[t] = acc;
                }
            }
        }
    }
    if (active && d_init) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int a = wr + 4 * t;
            if (a < NA)
                *reinterpret_cast<float4_t *>(d_init + ((int64_t)nh * DV + v0 + nn) * DK + 16 * a + 4 * jj) = s[t];
        }
    }
}

// ============================================================================
// B4: per (chunk row, head), every per-token gradient of the chunk.  Eight
// waves; wave w owns rows 16 (w % 4) .. + 15 of the chunk and half w / 4 of
// the key tiles.  The value dimension is walked in blocks of 16 columns: the
// products that sum over it (dP, dM, U = dO S, Z = dY S, W2 = V' dS_next)
// accumulate in registers.  The decay sums follow from them:
// dO_r . (Q S^T)_r = q_r . U_r, dY_r . X_r = k_r . Z_r and
// V'_r . (K dS_next^T)_r = k_r . W2_r.
// ============================================================================
// LDS of B4.  In the split form (bf16 inputs) Q and K are bf16 rows, which
// leaves room for two value-block buffers: one is staged while the other is
// read, one barrier per block.  After the loop dT / E and dP o Gamma overlay
// the first buffer and W / dK o follows.
template <int DK, bool SPL>
struct GradSmem {
    static constexpr int KP = DK + 4;       // Q, K rows (fp32)
    static constexpr int KB = DK + 8;       // Q, K rows (bf16, split form)
    static constexpr int CP = C + 4;        // C x C matrices
    static constexpr int BP = 16 + 4;       // value blocks [C][16] and transposed S / dS blocks [DK][16]
    static constexpr int NBUF = SPL ? 2 : 1;
    static constexpr int QK_FL = SPL ? C * KB / 2 : C * KP;
    static constexpr int off_q = 0;
    static constexpr int off_k = off_q + QK_FL;
    static constexpr int off_t = off_k + QK_FL;
    // one value-block buffer: S^T, dS^T, dO, Y, V', dV', dY blocks
    static constexpr int b_s = 0, b_ds = DK * BP, b_o = 2 * DK * BP, b_y = b_o + C * BP, b_vp = b_y + C * BP;
    static constexpr int b_dvp = b_vp + C * BP, b_dy = b_dvp + C * BP, VBUF = b_dy + C * BP;
    static constexpr int off_buf = off_t + C * CP;
    static constexpr int off_dt = off_buf;                // after the loop
    static constexpr int off_p = off_buf + C * CP;        // after the loop: dP o Gamma
    static constexpr int off_w = (off_buf + VBUF > off_p + C * CP) ? off_buf + VBUF : off_p + C * CP;  // W, later dK o
    static constexpr int END = (off_buf + NBUF * VBUF > off_w + C * CP) ? off_buf + NBUF * VBUF : off_w + C * CP;
    static constexpr int off_vec = END;                   // g, gamma, kappa, beta, dgamma, dkappa
    static constexpr int off_f = off_vec + 6 * C + 8;    // (after one <dS_next, S> part per wave)
    static constexpr int off_db = off_f + 4 * C;         // E L column sums, one row per row block
    static constexpr int floats = off_db + 6 * C;        // dbeta parts: [4][C] by row block, [2][C] by half
    static constexpr size_t bytes = sizeof(float) * floats;
    static_assert(off_buf % 4 == 0 && VBUF % 4 == 0, "16-byte aligned buffers");
    static_assert(bytes <= 160 * 1024, "one block per CU: at most the 160 KiB of LDS");
};

template <typename in_t, int DK>
__global__ __launch_bounds__(512) void bwd_grad_kernel(int H, int DV, int T, int cpr, int urows,
                                                       const int32_t *__restrict__ meta,
                                                       const int32_t *__restrict__ row_tok,
                                                       const int32_t *__restrict__ row_len,
                                                       const in_t *__restrict__ q, const in_t *__restrict__ k,
                                                       const float *__restrict__ d_o,
                                                       const float *__restrict__ ws_t,
                                                       const float *__restrict__ ws_p,
                                                       const float *__restrict__ ws_g,
                                                       const float *__restrict__ ws_vec,
                                                       const float *__restrict__ ws_ck,
                                                       const float *__restrict__ ws_ds,
                                                       const float *__restrict__ ws_y,
                                                       const float *__restrict__ ws_vp,
                                                       const float *__restrict__ ws_dvp, float *__restrict__ dq,
                                                       float *__restrict__ dk, const float *__restrict__ dv,
                                                       float *__restrict__ dla, float *__restrict__ dbeta) {
    constexpr bool SPL = SplitState<in_t>::value;
    using L = GradSmem<DK, SPL>;
    constexpr int KP = L::KP, KB = L::KB, CP = L::CP, BP = L::BP, NA = DK / 16, NH = NA / 2;
    extern __shared__ __align__(16) float smem[];
    float *sq = smem + L::off_q, *sk = smem + L::off_k, *st = smem + L::off_t, *sp = smem + L::off_p;
    const uint16_t *sqb = reinterpret_cast<const uint16_t *>(sq), *skb = reinterpret_cast<const uint16_t *>(sk);
    float *sw = smem + L::off_w;
    // Q and K element (r, c) as fp32, from fp32 or (split form) bf16 rows
    auto q_at = [&](int r, int c) { return SPL ? __uint_as_float((uint32_t)sqb[r * KB + c] << 16) : sq[r * KP + c]; };
    auto k_at = [&](int r, int c) { return SPL ? __uint_as_float((uint32_t)skb[r * KB + c] << 16) : sk[r * KP + c]; };
    float *vg = smem + L::off_vec, *vgam = vg + C, *vkap = vg + 2 * C, *vb = vg + 3 * C;
    float *vdgam = vg + 4 * C, *vdkap = vg + 5 * C;
    float *vgl = vg + 6 * C;   // per-wave parts of <dS_next, S>
    float *vF = smem + L::off_f;   // [4][C]
    // dbeta's parts, one slot per writer, summed in a fixed order at the end:
    // column sums of dM o T by the row block that formed them, and row sums
    // of dA o (Gamma o K K^T) by the half that formed them
    float *vdbc = smem + L::off_db, *vdbr = vdbc + 4 * C;
    if (!cpr && meta[1] != 0) return;
    const int nitems = (cpr ? urows : meta[0]) * H;
    int tid = threadIdx.x;
    // One value block's operands in registers.  S / dS_next block: lane tid
    // takes row tid % 16 and columns 4 (tid / 16 + 32 m) .. + 3, so the
    // transposed LDS stores of a wave hit consecutive banks; Y, V', dV':
    // element tid + 512 m of the C x 16 block.  dO and dY: element tid + 512 m
    // of C x PW columns, read when the first block of the PW columns is loaded.
    // In the split form (registers to spare) PW = 32, whole 128-byte lines for
    // a pair of blocks, and the lanes holding the second block's half keep it
    // until that block is staged; otherwise PW = 16.
    constexpr int NS = (DK / 4 + 31) / 32, PW = SPL ? 32 : 16, NP = PW / 8;
    struct VBlock {
        float4_t ga[NS], gb[NS];
        float go[NP], gdy[NP], gyv[2], gvp[2], gdvp[2];
    };
    auto load_block_of = [&](VBlock &B, int vb, int64_t it, int tok0, int len, int h) {
        const float *ck = ws_ck + it * DV * DK, *dsn = ws_ds + it * DV * DK;
        const float *gy = ws_y + it * C * DV, *gvp = ws_vp + it * C * DV, *gdvp = ws_dvp + it * C * DV;
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int cg = tid / 16 + 32 * m;
            if (cg < DK / 4) {
                const int r = tid % 16, c = 4 * cg;
                B.ga[m] = *reinterpret_cast<const float4_t *>(ck + (int64_t)(vb + r) * DK + c);
                B.gb[m] = *reinterpret_cast<const float4_t *>(dsn + (int64_t)(vb + r) * DK + c);
            }
        }
        if (vb % PW == 0) {   // the first block of the PW columns
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                const int e = tid + 512 * m, r = e / PW, c = e % PW;
                const bool in = r < len && vb + c < DV;
                const int64_t tv = ((int64_t)(tok0 + r) * H + h) * DV + vb + c;
                B.go[m] = in ? d_o[tv] : 0.f;
                B.gdy[m] = in ? dv[tv] : 0.f;
            }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int e = tid + 512 * m;
            const int64_t wv = (int64_t)vb * C + e;   // block-major: the C x 16 block is contiguous
            B.gyv[m] = gy[wv];
            B.gvp[m] = gvp[wv];
            B.gdvp[m] = gdvp[wv];
        }
    };
    // The operands an item starts with (its first value block, Q, K, T and
    // decay vectors), loaded into registers during the previous item's
    // post-loop steps: the block steps through items item0, item0 + grid, ...
    // Rows past the end re-read the last row and are zeroed when staged.
    constexpr int NQ = (C * DK + 4095) / 4096;
    VBlock VB;
    Raw8<in_t> qs[NQ], ks[NQ];
    float4_t ts[2];
    float vv0 = 0.f;
    auto item_span = [&](int item, int &tok0, int &len) {
        row_span(item / H, T, cpr, row_tok, row_len, tok0, len);
    };
    auto load_item = [&](int item) {
        int tok0, len;
        item_span(item, tok0, len);
        if (len == 0) return;   // (an empty sequence's row is skipped)
        const int h = item % H;
        const int64_t it = item;
        load_block_of(VB, 0, it, tok0, len, h);
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int idx = min(tid * 8 + 4096 * m, C * DK - 8), r = min(idx / DK, len - 1), c = idx % DK;
            const int64_t off = ((int64_t)(tok0 + r) * H + h) * DK + c;
            qs[m].load(q + off);
            ks[m].load(k + off);
        }
        const float *Tg = ws_t + it * C * C;
#pragma unroll
        for (int m = 0; m < 2; ++m) ts[m] = *reinterpret_cast<const float4_t *>(Tg + tid * 4 + 2048 * m);
        vv0 = ws_vec[it * kVecFloats + min(tid, 4 * C - 1)];
    };
    if ((int)blockIdx.x < nitems) load_item(blockIdx.x);
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    __syncthreads();   // the previous item's LDS contents are no longer read
    // (The lane index is re-issued per item so that the many addresses derived
    // from it are formed where they are used, not held across the item loop.)
    asm volatile("" : "+v"(tid));
    // Eight waves: wave w owns chunk rows 16 (w % 4) .. + 15; the two halves of
    // the block (w / 4) split the key-column tiles of U, Z, W2, dQ and dK, and
    // the decay-mask steps (half 0 holds dP, half 1 holds dM).
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wr = w & 3, half = w >> 2;
    const int l = tid & 63, nn = l & 15, jj = l >> 4;
    const int a0 = half * NH;
    const int h = item % H, next = item + (int)gridDim.x;
    int tok0, len;
    item_span(item, tok0, len);
    if (len == 0) {   // an empty sequence's row: it has no gradients
        if (next < nitems) load_item(next);
        continue;
    }
    const int64_t it64 = (int64_t)item;

    const float *Pg = ws_p + it64 * C * C, *Gg = ws_g + it64 * C * C;
    const int rw = 16 * wr;          // the wave's first chunk row
    // Sums over the value dimension, rows of the wave, key tiles a0 + a:
    //   U = dO S,  Z = dY S,  W2 = V' dS_next;  and tiles (wr, c <= wr) of
    //   dP = dO V'^T (half 0) or dM = dV' Y^T (half 1).
    float4_t au[NH], az[NH], aw[NH], dx[4];
#pragma unroll
    for (int a = 0; a < NH; ++a) au[a] = az[a] = aw[a] = zero4();
#pragma unroll
    for (int c = 0; c < 4; ++c) dx[c] = zero4();
    float pgl = 0.f;

    // The wave's decay-mask tiles: (wr, c) for c = 2 ci + half <= wr.  Their
    // (Q K^T) o Gamma and (K K^T) o Gamma, loaded here to land during the loop.
    float pvr[2][4], gvr[2][4];
#pragma unroll
    for (int ci = 0; ci < 2; ++ci)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 2 * ci + half, r = rw + 4 * jj + i, cc = 16 * c + nn;
            pvr[ci][i] = c <= wr ? Pg[r * C + cc] : 0.f;
            gvr[ci][i] = c <= wr ? Gg[r * C + cc] : 0.f;
        }

    auto load_block = [&](VBlock &B, int vb) { load_block_of(B, vb, it64, tok0, len, h); };
    // Write a loaded block into value-block buffer bb (S^T and dS_next^T
    // transposed: ss[c * BP + kk] = S[vb + kk][c]).
    auto stage_block = [&](const VBlock &B, int vb, float *bb) {
        float *ss = bb + L::b_s, *sds = bb + L::b_ds, *so = bb + L::b_o, *sy = bb + L::b_y;
        float *svp = bb + L::b_vp, *sdvp = bb + L::b_dvp, *sdy = bb + L::b_dy;
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int cg = tid / 16 + 32 * m;
            if (cg < DK / 4) {
                const int r = tid % 16, c = 4 * cg;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ss[(c + i) * BP + r] = B.ga[m][i];
                    sds[(c + i) * BP + r] = B.gb[m][i];
                }
                pgl += B.ga[m][0] * B.gb[m][0] + B.ga[m][1] * B.gb[m][1] + B.ga[m][2] * B.gb[m][2] +
                       B.ga[m][3] * B.gb[m][3];
            }
        }
        if (PW == 16 || ((tid >> 4) & 1) == ((vb >> 4) & 1)) {   // the lanes holding this block's part
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                const int e = tid + 512 * m, r = e / PW, c = e % 16;
                so[r * BP + c] = B.go[m];
                sdy[r * BP + c] = B.gdy[m];
            }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int e = tid + 512 * m, r = e / 16, c = e % 16;
            sy[r * BP + c] = B.gyv[m];
            svp[r * BP + c] = B.gvp[m];
            sdvp[r * BP + c] = B.gdvp[m];
        }
    };
    // The products of the block in buffer bb: one k-tile (its 16 value
    // columns), lane (n, j) supplying columns 4j .. 4j + 3.
    auto compute_block = [&](const float *bb) {
        const float *ss = bb + L::b_s, *sds = bb + L::b_ds, *so = bb + L::b_o, *sy = bb + L::b_y;
        const float *svp = bb + L::b_vp, *sdvp = bb + L::b_dvp, *sdy = bb + L::b_dy;
        const float *sxa = half ? sdvp : so, *sxb = half ? sy : svp;
        const float4_t ao = *reinterpret_cast<const float4_t *>(so + (rw + nn) * BP + 4 * jj);
        const float4_t ayv = *reinterpret_cast<const float4_t *>(sdy + (rw + nn) * BP + 4 * jj);
        const float4_t avp = *reinterpret_cast<const float4_t *>(svp + (rw + nn) * BP + 4 * jj);
        const float4_t ax = *reinterpret_cast<const float4_t *>(sxa + (rw + nn) * BP + 4 * jj);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c <= wr) {
                const float4_t bx = *reinterpret_cast<const float4_t *>(sxb + (16 * c + nn) * BP + 4 * jj);
#pragma unroll
                for (int i = 0; i < 4; ++i) mfma4(dx[c], ax[i], bx[i]);
            }
        }
#pragma unroll
        for (int a = 0; a < NH; ++a) {
            const float4_t bs = *reinterpret_cast<const float4_t *>(ss + (16 * (a0 + a) + nn) * BP + 4 * jj);
            const float4_t bd = *reinterpret_cast<const float4_t *>(sds + (16 * (a0 + a) + nn) * BP + 4 * jj);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mfma4(au[a], ao[i], bs[i]);
                mfma4(az[a], ayv[i], bs[i]);
                mfma4(aw[a], avp[i], bd[i]);
            }
        }
    };
    float *buf0 = smem + L::off_buf;
    // ---- stage Q, K, T and the vectors (loaded with the first value block
    // during the previous item) ----
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
        const int idx = tid * 8 + 4096 * m, r = idx / DK, c = idx % DK;
        if (SPL && idx < C * DK) {   // bf16 rows as they are
            if (r >= len) {
                qs[m].zero();
                ks[m].zero();
            }
            qs[m].store_lds(reinterpret_cast<in_t *>(sq) + r * KB + c);
            ks[m].store_lds(reinterpret_cast<in_t *>(sk) + r * KB + c);
        } else if (idx < C * DK) {
            float xq[8], xk[8];
            qs[m].to_f32(xq);
            ks[m].to_f32(xk);
            if (r >= len)
#pragma unroll
                for (int e = 0; e < 8; ++e) xq[e] = xk[e] = 0.f;
            *reinterpret_cast<float4_t *>(sq + r * KP + c) = float4_t{xq[0], xq[1], xq[2], xq[3]};
            *reinterpret_cast<float4_t *>(sq + r * KP + c + 4) = float4_t{xq[4], xq[5], xq[6], xq[7]};
            *reinterpret_cast<float4_t *>(sk + r * KP + c) = float4_t{xk[0], xk[1], xk[2], xk[3]};
            *reinterpret_cast<float4_t *>(sk + r * KP + c + 4) = float4_t{xk[4], xk[5], xk[6], xk[7]};
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int e = tid * 4 + 2048 * m, r = e / C, c = e % C;
        *reinterpret_cast<float4_t *>(st + r * CP + c) = ts[m];
    }
    if (tid < 4 * C) vg[tid] = vv0;
    if (tid < 2 * C) vdgam[tid] = 0.f;   // dgamma and dkappa: two addends per slot
    if (tid < 4 * C) vF[tid] = 0.f;
    if constexpr (L::NBUF == 2) {   // block 0 staged with the rest
        stage_block(VB, 0, buf0);
        load_block(VB, min(16, DV - 16));
    }
    __syncthreads();

    if constexpr (L::NBUF == 2) {
        // Block i is read from buffer i % 2 while block i + 1 is staged into
        // the other; the barrier after both makes block i + 1 visible and
        // frees buffer i % 2 for block i + 2.
        for (int vb0 = 0, i = 0; vb0 < DV; vb0 += 16, ++i) {
            compute_block(buf0 + (i & 1) * L::VBUF);
            if (vb0 + 16 < DV) {
                stage_block(VB, vb0 + 16, buf0 + ((i + 1) & 1) * L::VBUF);
                load_block(VB, min(vb0 + 32, DV - 16));   // (the last blocks load themselves again)
            }
            __syncthreads();
        }
    } else {
        for (int vb0 = 0; vb0 < DV; vb0 += 16) {
            __syncthreads();   // the previous block is no longer read
            stage_block(VB, vb0, buf0);
            if (vb0 + 16 < DV) load_block(VB, vb0 + 16);
            __syncthreads();
            compute_block(buf0);
        }
    }

    // ---- decay sums: dgamma_r = q_r . U_r - k_r . Z_r,  dkappa_r = k_r . W2_r ----
    // Each half adds its key tiles' part to a zeroed slot: two addends, so
    // the result does not depend on their order.
    {
        float pg[4] = {0.f, 0.f, 0.f, 0.f}, pk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int a = 0; a < NH; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rw + 4 * jj + i, c = 16 * (a0 + a) + nn;
                const float qv = q_at(r, c), kv = k_at(r, c);
                pg[i] += qv * au[a][i] - kv * az[a][i];
                pk[i] += kv * aw[a][i];
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float g1 = row16_sum(pg[i]), k1 = row16_sum(pk[i]);
            if (nn == 0) {
                atomicAdd(&vdgam[rw + 4 * jj + i], g1);
                atomicAdd(&vdkap[rw + 4 * jj + i], k1);
            }
        }
    }
    // dQ and dK rows of the wave so far: diag(gamma) U and -diag(gamma) Z + diag(kappa) W2
    float4_t accq[NH], acck[NH];
#pragma unroll
    for (int a = 0; a < NH; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rw + 4 * jj + i;
            accq[a][i] = vgam[r] * au[a][i];
            acck[a][i] = vkap[r] * aw[a][i] - vgam[r] * az[a][i];
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) pgl += __shfl_xor(pgl, o, 64);
    if (l == 0) vgl[w] = pgl;
    __syncthreads();
    float *sdt = smem + L::off_dt;   // [C][CP]
    if (half) {
        // dT = dM diag(beta) on the lower triangle (zero above), into the
        // value-loop area; dbeta's first part, column sums of dM o T
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float cs = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rw + 4 * jj + i, cc = 16 * c + nn;
                const bool in = c <= wr && cc <= r;
                sdt[r * CP + cc] = in ? dx[c][i] * vb[cc] : 0.f;
                cs += in ? dx[c][i] * st[r * CP + cc] : 0.f;
            }
            if (c <= wr) {
                cs += __shfl_xor(cs, 16, 64);
                cs += __shfl_xor(cs, 32, 64);
                if (jj == 0) vdbc[wr * C + 16 * c + nn] = cs;
            }
        }
    } else {
        // dP on the lower triangle (zero above)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rw + 4 * jj + i, cc = 16 * c + nn;
                sp[r * CP + cc] = c <= wr && cc <= r ? dx[c][i] : 0.f;
            }
    }
    __syncthreads();
    // W = T^T dT, rows of the wave, column blocks 2 half and 2 half + 1 (one
    // read of T per k-tile for both).  T is lower triangular, so k-tiles
    // before the wave's rows add nothing.
    {
        const int c0 = 2 * half;
        float4_t wt0 = zero4(), wt1 = zero4();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            if (kt < wr) continue;
            float ta[4], b0[4], b1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 16 * kt + 4 * jj + i;
                ta[i] = st[kk * CP + rw + nn];
                b0[i] = sdt[kk * CP + 16 * c0 + nn];
                b1[i] = sdt[kk * CP + 16 * c0 + 16 + nn];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mfma4(wt0, ta[i], b0[i]);
                mfma4(wt1, ta[i], b1[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sw[(rw + 4 * jj + i) * CP + 16 * c0 + nn] = wt0[i];
            sw[(rw + 4 * jj + i) * CP + 16 * c0 + 16 + nn] = wt1[i];
        }
    }
    __syncthreads();
    // dA = -W T^T on the wave's tiles (T^T is upper triangular: k-tiles up to
    // c); with K K^T, Q K^T and Gamma form dbeta's second part, dK o, dP o
    // Gamma and E = dGamma o Gamma.
    float4_t dkk[2];
    float dbr[4] = {0.f, 0.f, 0.f, 0.f};   // the wave's row sums for dbeta, tile by tile
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
        const int c = 2 * ci + half;
        dkk[ci] = zero4();
        if (c > wr) continue;
        float4_t da = zero4();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            if (kt > c) continue;
            const float4_t wa = *reinterpret_cast<const float4_t *>(sw + (rw + nn) * CP + 16 * kt + 4 * jj);
            const float4_t tb = *reinterpret_cast<const float4_t *>(st + (16 * c + nn) * CP + 16 * kt + 4 * jj);
#pragma unroll
            for (int i = 0; i < 4; ++i) mfma4(da, -wa[i], tb[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rw + 4 * jj + i, cc = 16 * c + nn;
            const float gm = cc <= r ? expf(vg[r] - vg[cc]) : 0.f;
            const float pv = pvr[ci][i], gv = gvr[ci][i];
            const float dav = cc < r ? da[i] : 0.f;
            const float db2 = dav * gv;
            const float dB = vb[r] * dav;
            dkk[ci][i] = dB * gm;
            const float dpv = sp[r * CP + cc];   // zero above the diagonal
            // E = dGamma o Gamma with dGamma = dP o Q K^T + dB o K K^T
            const float dgg = dpv * pv + dB * gv;
            sp[r * CP + cc] = dpv * gm;         // dP o Gamma
            dbr[i] += row16_sum(db2);
            sdt[r * CP + cc] = cc < r ? dgg : 0.f;   // strictly lower; the upper tiles hold dT's zeros
        }
    }
    if (nn == 0)   // every wave writes its rows' slot, zero where it had no tile
#pragma unroll
        for (int i = 0; i < 4; ++i) vdbr[half * C + rw + 4 * jj + i] = dbr[i];
    __syncthreads();
    // dK o (strictly lower) into sw (W is no longer needed)
#pragma unroll
    for (int ci = 0; ci < 2; ++ci)
#pragma unroll
        for (int i = 0; i < 4; ++i) sw[(rw + 4 * jj + i) * CP + 16 * (2 * ci + half) + nn] = dkk[ci][i];
    // The sums of E = dGamma o Gamma that dlog alpha needs,
    //   F_i = sum_{r >= i} sum_{c < i} E_rc = sum_{r >= i} (E L)_ri,  L_ci = [c < i],
    // one column tile (wr, c) of E L per wave tile c = 2 ci + half <= wr (the
    // rows r >= i of a column block c lie in row blocks >= c); L is formed in
    // registers, E is strictly lower, so k-tiles up to c.  Each tile's masked
    // column sums go to its own slot of vF, added in a fixed order below.
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
        const int c = 2 * ci + half;
        if (c > wr) continue;
        float4_t el = zero4();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            if (kt > c) continue;
            const float4_t ea = *reinterpret_cast<const float4_t *>(sdt + (rw + nn) * CP + 16 * kt + 4 * jj);
#pragma unroll
            for (int i = 0; i < 4; ++i) mfma4(el, ea[i], 16 * kt + 4 * jj + i < 16 * c + nn ? 1.f : 0.f);
        }
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) cs += rw + 4 * jj + i >= 16 * c + nn ? el[i] : 0.f;
        cs += __shfl_xor(cs, 16, 64);
        cs += __shfl_xor(cs, 32, 64);
        if (jj == 0) vF[wr * C + 16 * c + nn] = cs;
    }
    __syncthreads();
    // Start the next item's loads, to land during this item's last products
    // (late, where fewer registers are live).
    if (next < nitems) load_item(next);
    // dQ += (dP o Gamma) K;  dK += (dP o Gamma)^T Q + (dK o + dK o^T) K.  The
    // row-side operands do not depend on the key tile: read once per k-tile.
    // dP o Gamma is lower triangular: k-tiles up to the wave's rows for dQ,
    // from them on for dK.
    if constexpr (SplitState<in_t>::value) {
        // bf16 inputs: K and Q are bf16 rows, so each product takes the row-side
        // operand as three exact bf16 terms, per 32-wide k slice.
        auto split8 = [](const float (&x)[8], uint4 (&t)[3]) {
            uint2 h0, m0, l0, h1, m1, l1;
            split3(float4_t{x[0], x[1], x[2], x[3]}, h0, m0, l0);
            split3(float4_t{x[4], x[5], x[6], x[7]}, h1, m1, l1);
            t[0] = uint4{h0.x, h0.y, h1.x, h1.y};
            t[1] = uint4{m0.x, m0.y, m1.x, m1.y};
            t[2] = uint4{l0.x, l0.y, l1.x, l1.y};
        };
        // Every slice takes all three products: where a slice lies wholly above
        // (dQ) or below (dK) the wave's rows, dP o Gamma is zero there and adds
        // nothing.
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks) {
            float x1[8], x2[8], x3[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kx = 32 * ks + 8 * jj + e;
                x1[e] = sp[(rw + nn) * CP + kx];
                x2[e] = sp[kx * CP + rw + nn];
                x3[e] = sw[(rw + nn) * CP + kx] + sw[kx * CP + rw + nn];
            }
            uint4 t1[3], t2[3], t3[3];
            split8(x1, t1);
            split8(x2, t2);
            split8(x3, t3);
#pragma unroll
            for (int a = 0; a < NH; ++a) {
                const int ka = 16 * (a0 + a);
                const uint4 kb = lds_col8_b16(skb, KB, 32 * ks, ka, nn, jj);   // columns ka .. of K and Q
                const uint4 qb = lds_col8_b16(sqb, KB, 32 * ks, ka, nn, jj);
#pragma unroll
                for (int term = 0; term < 3; ++term) {
                    mfma_bf16(acck[a], t3[term], kb);
                    mfma_bf16(accq[a], t1[term], kb);
                    mfma_bf16(acck[a], t2[term], qb);
                }
            }
        }
    } else {
        // fp32 products, every k-tile issued (as in the split form): where a
        // tile lies above (dQ) or below (dK) the wave's rows dP o Gamma is zero.
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const float4_t a1 = *reinterpret_cast<const float4_t *>(sp + (rw + nn) * CP + 16 * kt + 4 * jj);
            const float4_t w1 = *reinterpret_cast<const float4_t *>(sw + (rw + nn) * CP + 16 * kt + 4 * jj);
            float a2[4], a3[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kx = 16 * kt + 4 * jj + i;
                a2[i] = sp[kx * CP + rw + nn];
                a3[i] = w1[i] + sw[kx * CP + rw + nn];
            }
#pragma unroll
            for (int a = 0; a < NH; ++a) {
                const int ka = 16 * (a0 + a);
                float bk[4], bq[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kx = 16 * kt + 4 * jj + i;
                    bk[i] = sk[kx * KP + ka + nn];
                    bq[i] = sq[kx * KP + ka + nn];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) mfma4(acck[a], a3[i], bk[i]);
#pragma unroll
                for (int i = 0; i < 4; ++i) mfma4(accq[a], a1[i], bk[i]);
#pragma unroll
                for (int i = 0; i < 4; ++i) mfma4(acck[a], a2[i], bq[i]);
            }
        }
    }
#pragma unroll
    for (int a = 0; a < NH; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rw + 4 * jj + i;
            if (r < len) {
                const int64_t off = ((int64_t)(tok0 + r) * H + h) * DK + 16 * (a0 + a) + nn;
                dq[off] = accq[a][i];
                dk[off] = acck[a][i];
            }
        }
    // dlog alpha_i is the sum over r >= i of dg_r.  Written out term by term
    // it is sum_{r>=i} gamma_r dgamma_r + sum_{r<i} kappa_r dkappa_r
    // + gamma_last <dS_next, S> + F_i: every term already carries its decay
    // factor, so a tiny gradient (strong decay) is not the difference of large
    // partial sums.  Wave 0, lane i: the suffix sum as a scan over the
    // reversed lanes, the exclusive prefix as the scan shifted by one lane.
    if (w == 0) {
        const int i = l;
        const float sfx_in = vdgam[C - 1 - l] * vgam[C - 1 - l];
        const float sfx = __shfl(wave_inclusive_scan(sfx_in), C - 1 - l, 64);   // sum_{r >= i}
        const float pin = wave_inclusive_scan(vdkap[l] * vkap[l]);
        float pre = __shfl_up(pin, 1, 64);                                      // sum_{r < i}
        if (l == 0) pre = 0.f;
        float gl = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) gl += vgl[u];
        const float f = ((vF[i] + vF[C + i]) + vF[2 * C + i]) + vF[3 * C + i];
        if (i < len) {
            const int64_t th = (int64_t)(tok0 + i) * H + h;
            dla[th] = gl * vgam[len - 1] + sfx + pre + f;
            // column-sum parts of the row blocks at or below column i's block, then the row sums
            float db = 0.f;
            for (int b = i / 16; b < 4; ++b) db += vdbc[b * C + i];
            dbeta[th] = (db + vdbr[i]) + vdbr[C + i];
        }
    }
    }   // items
}

// ============================================================================
// Host side
// ============================================================================
namespace {

template <typename K>
hipError_t bwd_allow_smem(K kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

// Compute units of the current device (cached after the first query).
int bwd_cu_count() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus = n;
    }
    return cus;
}

int bwd_cpr(const ChunkArgs &a) { return a.cu_seqlens ? 0 : (a.T + C - 1) / C + (a.T == 0); }

template <typename in_t, int DK>
hipError_t launch_bwd_dk(const ChunkArgs &a, const BwdArgs &g, const BwdWorkspace &w, hipStream_t st) {
    char *ws = static_cast<char *>(a.workspace);
    const int32_t *meta = reinterpret_cast<const int32_t *>(ws + w.fwd.off_meta);
    const int32_t *cu_ws = reinterpret_cast<const int32_t *>(ws + w.fwd.off_cu);
    const int32_t *row0 = reinterpret_cast<const int32_t *>(ws + w.fwd.off_row0);
    const int32_t *rtok = reinterpret_cast<const int32_t *>(ws + w.fwd.off_rowtok);
    const int32_t *rlen = reinterpret_cast<const int32_t *>(ws + w.fwd.off_rowlen);
    float *wt = reinterpret_cast<float *>(ws + w.off_t), *wp = reinterpret_cast<float *>(ws + w.off_p);
    float *wg = reinterpret_cast<float *>(ws + w.off_gk);
    float *wv = reinterpret_cast<float *>(ws + w.off_vec), *wck = reinterpret_cast<float *>(ws + w.off_ck);
    float *wds = reinterpret_cast<float *>(ws + w.off_ds);
    float *wy = reinterpret_cast<float *>(ws + w.off_y), *wvp = reinterpret_cast<float *>(ws + w.off_vp);
    float *wdvp = reinterpret_cast<float *>(ws + w.off_dvp);
    auto *q = static_cast<const in_t *>(a.q);
    auto *k = static_cast<const in_t *>(a.k);
    auto *v = static_cast<const in_t *>(a.v);
    const int cpr = bwd_cpr(a);
    const int urows = cpr ? (int)w.fwd.max_rows : 0;
    const int64_t items = w.fwd.max_rows * a.H;
    const int nvt = a.dv / 16;
    const int NH = a.N * a.H;
    const int64_t chains = (int64_t)NH * nvt, heads8 = (NH + 7) / 8 * 8;
    hipError_t e;
    if (items > 0) {
        ProfScope prof("gdn_bwd_prep", st);
        bwd_prep_kernel<in_t, DK><<<dim3((unsigned)items), dim3(64), 0, st>>>(a.H, a.T, cpr, urows, meta, rtok, rlen,
                                                                             q, k, a.log_alpha, a.beta, wt, wp, wg, wv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (chains > 0) {
        {
            const size_t sb = PassSmem<DK, SplitState<in_t>::value>::bytes_fwd;
            auto kern = bwd_fwd_pass_kernel<in_t, DK>;
            if ((e = bwd_allow_smem(kern, sb)) != hipSuccess) return e;
            ProfScope prof("gdn_bwd_fwd_pass", st);
            kern<<<dim3((unsigned)(heads8 * nvt)), dim3(256), sb, st>>>(NH, a.H, a.dv, a.T, cpr, nvt, meta, cu_ws,
                                                                        row0, rtok, rlen, k, v, wt, wv,
                                                                        a.init_state, wck, wy, wvp);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        {
            const size_t sb = RevSmem<DK, SplitState<in_t>::value>::bytes;
            auto kern = bwd_rev_pass_kernel<in_t, DK>;
            if ((e = bwd_allow_smem(kern, sb)) != hipSuccess) return e;
            ProfScope prof("gdn_bwd_rev_pass", st);
            const unsigned grid = (unsigned)(heads8 * ((nvt + 1) / 2));
            kern<<<dim3(grid), dim3(512), sb, st>>>(NH, a.H, a.dv, a.T, cpr, nvt, meta, cu_ws, row0, rtok, rlen, q, k,
                                                    g.d_o, wt, wp, wv, g.d_final, wds, wdvp, g.dv, g.d_init);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if (items > 0) {
        using L = GradSmem<DK, SplitState<in_t>::value>;
        auto kern = bwd_grad_kernel<in_t, DK>;
        if ((e = bwd_allow_smem(kern, L::bytes)) != hipSuccess) return e;
        // A block per resident slot, each stepping through the items, so the
        // next item's first loads overlap the current item's last steps.
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), 512,
                                                         L::bytes) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        const int64_t grid = std::min<int64_t>(items, (int64_t)per_cu * bwd_cu_count());
        ProfScope prof("gdn_bwd_grad", st);
        kern<<<dim3((unsigned)grid), dim3(512), L::bytes, st>>>(a.H, a.dv, a.T, cpr, urows, meta, rtok, rlen, q, k,
                                                                 g.d_o, wt, wp, wg, wv, wck, wds, wy, wvp, wdvp, g.dq,
                                                                 g.dk, g.dv, g.dlog_alpha, g.dbeta);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename in_t>
hipError_t launch_bwd_typed(const ChunkArgs &a, const BwdArgs &g, const BwdWorkspace &w, hipStream_t st) {
    switch (a.dk) {
    case 32: return launch_bwd_dk<in_t, 32>(a, g, w, st);
    case 64: return launch_bwd_dk<in_t, 64>(a, g, w, st);
    case 128: return launch_bwd_dk<in_t, 128>(a, g, w, st);
    }
    return hipErrorInvalidValue;
}

// ============================================================================
// q/k L2 normalisation (GDN_QK_L2NORM).  The forward pass evaluates the rule
// on q^ = q / ||q|| and k^ = k / ||k|| per (token, head), a zero row staying
// zero (Gated Delta Networks paper, section 3.4: the token mixer block
// normalises q and k).  The backward pass runs the kernels above on q^, k^
// as fp32 rows (v widened to fp32 beside them: the kernels take one input
// type) and then maps the gradients of q^ and k^ through the normalisation,
//   dx = (dx^ - x^ (x^ . dx^)) / ||x||        (0 for a zero row),
// the derivative of x / ||x||.  LPR = DK / 8 lanes share one (token, head)
// row, 8 elements each; the row sums go by xor shuffles within those lanes.
// ============================================================================
template <typename in_t, int DK>
__global__ __launch_bounds__(256) void bwd_norm_in_kernel(int64_t rows, int DV, const in_t *__restrict__ q,
                                                          const in_t *__restrict__ k, const in_t *__restrict__ v,
                                                          float *__restrict__ qh, float *__restrict__ kh,
                                                          float *__restrict__ v32, float *__restrict__ rqk) {
    constexpr int LPR = DK / 8, RPB = 256 / LPR;
    const int sub = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (row >= rows) return;   // the lanes of a row leave together
    const int64_t e0 = row * DK + 8 * sub;
    Raw8<in_t> rq, rk;
    rq.load(q + e0);
    rk.load(k + e0);
    float xq[8], xk[8];
    rq.to_f32(xq);
    rk.to_f32(xk);
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sq = fmaf(xq[e], xq[e], sq);
        sk = fmaf(xk[e], xk[e], sk);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) {
        sq += __shfl_xor(sq, m, 64);
        sk += __shfl_xor(sk, m, 64);
    }
    const float fq = sq > 0.f ? rsqrtf(sq) : 0.f, fk = sk > 0.f ? rsqrtf(sk) : 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<float4_t *>(qh + e0 + 4 * h) =
            float4_t{fq * xq[4 * h], fq * xq[4 * h + 1], fq * xq[4 * h + 2], fq * xq[4 * h + 3]};
        *reinterpret_cast<float4_t *>(kh + e0 + 4 * h) =
            float4_t{fk * xk[4 * h], fk * xk[4 * h + 1], fk * xk[4 * h + 2], fk * xk[4 * h + 3]};
    }
    if (sub == 0) *reinterpret_cast<float2 *>(rqk + 2 * row) = make_float2(fq, fk);
    for (int c = sub; c < DV; c += LPR) v32[row * DV + c] = to_f32(v[row * DV + c]);
}

template <int DK>
__global__ __launch_bounds__(256) void bwd_norm_out_kernel(int64_t rows, int cpr, const int32_t *__restrict__ meta,
                                                           const float *__restrict__ qh, const float *__restrict__ kh,
                                                           const float *__restrict__ rqk, float *__restrict__ dq,
                                                           float *__restrict__ dk) {
    constexpr int LPR = DK / 8, RPB = 256 / LPR;
    if (!cpr && meta[1] != 0) return;   // malformed cu_seqlens: no gradient was written
    const int sub = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (row >= rows) return;
    const int64_t e0 = row * DK + 8 * sub;
    const float2 f = *reinterpret_cast<const float2 *>(rqk + 2 * row);
    auto map = [&](const float *xh, float *d, float fx) {
        float4_t x[2], g[2];
        float dot = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            x[h] = *reinterpret_cast<const float4_t *>(xh + e0 + 4 * h);
            g[h] = *reinterpret_cast<const float4_t *>(d + e0 + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) dot = fmaf(x[h][i], g[h][i], dot);
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float4_t r;
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = fx * fmaf(-x[h][i], dot, g[h][i]);
            *reinterpret_cast<float4_t *>(d + e0 + 4 * h) = r;
        }
    };
    map(qh, dq, f.x);
    map(kh, dk, f.y);
}

template <typename in_t>
hipError_t launch_bwd_norm_in(const ChunkArgs &a, const BwdWorkspace &w, hipStream_t st) {
    char *ws = static_cast<char *>(a.workspace);
    const int64_t rows = (int64_t)a.B * a.T * a.H;
    auto go = [&](auto kern, int lpr) {
        const int64_t rpb = 256 / lpr;
        ProfScope prof("gdn_bwd_norm_in", st);
        kern<<<dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, st>>>(
            rows, a.dv, static_cast<const in_t *>(a.q), static_cast<const in_t *>(a.k),
            static_cast<const in_t *>(a.v), reinterpret_cast<float *>(ws + w.off_qh),
            reinterpret_cast<float *>(ws + w.off_kh), reinterpret_cast<float *>(ws + w.off_v32),
            reinterpret_cast<float *>(ws + w.off_rqk));
        return hipGetLastError();
    };
    switch (a.dk) {
    case 32: return go(bwd_norm_in_kernel<in_t, 32>, 4);
    case 64: return go(bwd_norm_in_kernel<in_t, 64>, 8);
    case 128: return go(bwd_norm_in_kernel<in_t, 128>, 16);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_norm_out(const ChunkArgs &a, const BwdArgs &g, const BwdWorkspace &w, hipStream_t st) {
    char *ws = static_cast<char *>(a.workspace);
    const int64_t rows = (int64_t)a.B * a.T * a.H;
    auto go = [&](auto kern, int lpr) {
        const int64_t rpb = 256 / lpr;
        ProfScope prof("gdn_bwd_norm_out", st);
        kern<<<dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, st>>>(
            rows, bwd_cpr(a), reinterpret_cast<const int32_t *>(ws + w.fwd.off_meta),
            reinterpret_cast<const float *>(ws + w.off_qh), reinterpret_cast<const float *>(ws + w.off_kh),
            reinterpret_cast<const float *>(ws + w.off_rqk), g.dq, g.dk);
        return hipGetLastError();
    };
    switch (a.dk) {
    case 32: return go(bwd_norm_out_kernel<32>, 4);
    case 64: return go(bwd_norm_out_kernel<64>, 8);
    case 128: return go(bwd_norm_out_kernel<128>, 16);
    }
    return hipErrorInvalidValue;
}

}  // namespace

static size_t bwd_align256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdWorkspace chunk_bwd_workspace_layout(int32_t B, int32_t T, int32_t N, bool packed, int32_t H, int32_t dk,
                                        int32_t dv, bool qk_norm) {
    BwdWorkspace w{};
    w.fwd = chunk_workspace_layout(B, T, N, packed, H, DT_FP32, dk, dv);
    const size_t items = (size_t)w.fwd.max_rows * H;
    size_t off = bwd_align256(w.fwd.off_g);   // only the table part of the forward layout is used
    w.off_t = off;   off = bwd_align256(off + sizeof(float) * items * C * C);
    w.off_p = off;   off = bwd_align256(off + sizeof(float) * items * C * C);
    w.off_gk = off;  off = bwd_align256(off + sizeof(float) * items * C * C);
    w.off_vec = off; off = bwd_align256(off + sizeof(float) * items * kVecFloats);
    w.off_ck = off;  off = bwd_align256(off + sizeof(float) * items * (size_t)dv * dk);
    w.off_ds = off;  off = bwd_align256(off + sizeof(float) * items * (size_t)dv * dk);
    w.off_y = off;   off = bwd_align256(off + sizeof(float) * items * C * (size_t)dv);
    w.off_vp = off;  off = bwd_align256(off + sizeof(float) * items * C * (size_t)dv);
    w.off_dvp = off; off = bwd_align256(off + sizeof(float) * items * C * (size_t)dv);
    if (qk_norm) {   // q^, k^ and v as fp32 rows, and the two normalisation factors per (token, head)
        const size_t th = (size_t)B * T * H;
        w.off_qh = off;  off = bwd_align256(off + sizeof(float) * th * dk);
        w.off_kh = off;  off = bwd_align256(off + sizeof(float) * th * dk);
        w.off_v32 = off; off = bwd_align256(off + sizeof(float) * th * dv);
        w.off_rqk = off; off = bwd_align256(off + sizeof(float) * th * 2);
    }
    w.total = off;
    return w;
}

hipError_t launch_chunk_bwd(const ChunkArgs &a, const BwdArgs &g, hipStream_t st) {
    const bool packed = a.cu_seqlens != nullptr;
    const bool qk_norm = (a.flags & kFlagQkL2Norm) != 0;
    const BwdWorkspace w = chunk_bwd_workspace_layout(a.B, a.T, a.N, packed, a.H, a.dk, a.dv, qk_norm);
    char *ws = static_cast<char *>(a.workspace);
    if (packed) {
        hipError_t e = launch_chunk_table(a.N, a.T, a.cu_seqlens, reinterpret_cast<int32_t *>(ws + w.fwd.off_meta),
                                          reinterpret_cast<int32_t *>(ws + w.fwd.off_cu),
                                          reinterpret_cast<int32_t *>(ws + w.fwd.off_row0),
                                          reinterpret_cast<int32_t *>(ws + w.fwd.off_rowtok),
                                          reinterpret_cast<int32_t *>(ws + w.fwd.off_rowlen), 0, nullptr, nullptr,
                                          nullptr, st);
        if (e != hipSuccess) return e;
    }
    if (qk_norm) {
        hipError_t e = a.in_dtype == DT_FP32   ? launch_bwd_norm_in<float>(a, w, st)
                       : a.in_dtype == DT_BF16 ? launch_bwd_norm_in<bf16_t>(a, w, st)
                                               : launch_bwd_norm_in<_Float16>(a, w, st);
        if (e != hipSuccess) return e;
        ChunkArgs an = a;
        an.q = ws + w.off_qh;
        an.k = ws + w.off_kh;
        an.v = ws + w.off_v32;
        an.in_dtype = DT_FP32;
        an.flags = 0;
        e = launch_bwd_typed<float>(an, g, w, st);
        if (e != hipSuccess) return e;
        return launch_bwd_norm_out(a, g, w, st);
    }
    switch (a.in_dtype) {
    case DT_FP32: return launch_bwd_typed<float>(a, g, w, st);
    case DT_BF16: return launch_bwd_typed<bf16_t>(a, g, w, st);
    case DT_FP16: return launch_bwd_typed<_Float16>(a, g, w, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
