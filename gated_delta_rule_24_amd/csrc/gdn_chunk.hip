// Chunkwise-parallel forward pass of the gated delta rule on gfx950.
//
// Per (sequence, head) the tokens are cut into chunks of C = 64 rows
// (row-stacked blocks Q, K in R^{C x dk}, V in R^{C x dv}).  With the state S
// (dv x dk) at the chunk start, the chunk algorithm of the Gated Delta
// Networks paper (section 3.3; paper-notes blog, "Hardware-Efficient
// Chunkwise Training", summary (4), which derives the decay mask in the
// output term) is
//
//   g_r      = sum_{i <= r} log alpha_i            (gamma^r = exp g_r)
//   Gamma_ri = exp(g_r - g_i) for i <= r, else 0   (masked before exp)
//   A        = strictLower(diag(beta) (Gamma o K K^T))
//   T        = (I + A)^{-1}                       (UT transform)
//   W        = T diag(beta) diag(gamma) K,   U = T diag(beta) V
//   V'       = U - W S^T
//   O        = diag(gamma) Q S^T + (Q K^T o Gamma) V'
//   S_next   = gamma^C S + V'^T diag(exp(g_C - g_r)) K
//
// The kernels use the same algebra regrouped:
//   V' = M Y,  M = T diag(beta),  Y = V - diag(gamma) (K S^T),
// i.e. W S^T is formed as M (diag(gamma) K S^T) instead of materialising W,
// which saves a C x C x dk product per chunk and keeps the per-chunk matrices
// handed from G1 to G2 at C x C size; and V' itself is never formed: the
// update takes diag(kappa) V' = (diag(kappa) M) Y and the output (P o
// Gamma-masked) V' = (P M) Y, with diag(kappa) M and P M made by G1.
//
// Kernels (all launched on the caller's stream):
//   G0 chunk_table_kernel  packed batches only, one block: validates
//                          cu_seqlens and lays out the (sequence, chunk)
//                          rows.  Equal-length batches derive a row's span
//                          from its index.
//   G1 chunk_prep_kernel   one wave per (chunk row, head), fully parallel:
//                          cumulative log-decay g, the decay-masked Q K^T
//                          block P, A, T = (I + A)^{-1} (diagonal 16x16
//                          blocks by back substitution, the rest by blocked
//                          products), M = T diag(beta) and the products
//                          diag(kappa) M and P M, which it writes to the
//                          workspace with the decay factors.
//   G2 chunk_state_kernel  one block per (sequence, head, value tile), serial
//                          over the sequence's chunks.  Each wave owns 16
//                          value columns and keeps its slice of S^T in
//                          registers (fp32 MFMA accumulators) for the whole
//                          sequence.  Per chunk:  X = [Q; K] S^T,
//                          Y = V - diag(gamma) X_K,
//                          O = diag(gamma) X_Q + (P M) Y,
//                          S^T <- gamma^C S^T + K^T ((diag(kappa) M) Y).
//                          Accumulator tiles feed the next product as B
//                          operands directly (see gdn_device.h), so only the
//                          shared Q, K, K^T, M, P blocks go through LDS.
#include "gdn_device.h"
#include "gdn_launch.h"

#include <stdlib.h>

#include <algorithm>
#include <type_traits>

namespace gdn {

constexpr int C = kChunk;

__device__ __forceinline__ void store_out(void *o, int64_t idx, int odt, float val) {
    if (odt == DT_FP32)
        static_cast<float *>(o)[idx] = val;
    else if (odt == DT_BF16)
        static_cast<bf16_t *>(o)[idx] = from_f32<bf16_t>(val);
    else
        static_cast<_Float16 *>(o)[idx] = (_Float16)val;
}

// Store 8 fp32 values as operands (two 4-element LDS writes).
template <typename OP>
__device__ __forceinline__ void lds_store8(OP *p, const float (&x)[8]) {
    using M = Mma<OP>;
    *reinterpret_cast<typename M::frag *>(p) = M::cvt(float4_t{x[0], x[1], x[2], x[3]});
    *reinterpret_cast<typename M::frag *>(p + 4) = M::cvt(float4_t{x[4], x[5], x[6], x[7]});
}

// ============================================================================
// G0: chunk table of a packed batch (cu_seqlens given).
//   meta[0] = number of rows, meta[1] = cu_seqlens error code (0 = valid),
//   meta[2] = number of segment units (segmented state pass only)
//   cu_ws[N+1] = token offsets, row0[N] = first row of each sequence,
//   row_tok / row_len = token start and length of each row.
// With seg_chunks > 0 each sequence's chunks are also cut into segments of
// seg_chunks chunks (at least one segment, so an empty sequence still carries
// its initial state to its final state): seg_first[n] / seg_cnt[n] = first
// unit and unit count of sequence n, seg_tab[2u], seg_tab[2u + 1] = (n, s).
// A batch of equal-length sequences needs no table: G1 and G2 derive a row's
// span from its index (row_span, gdn_launch.h) and G0 is not launched.
// ============================================================================

// Exclusive prefix sums of cnt(n), n < N, into out[n] by one 256-thread block;
// returns the total.  Every thread of the block must call it.
template <typename F>
__device__ int block_exclusive_scan(int N, F cnt, int32_t *__restrict__ out, int *s_scan, int *s_offset) {
    const int tid = threadIdx.x;
    if (tid == 0) *s_offset = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + tid;
        const int c = n < N ? cnt(n) : 0;
        s_scan[tid] = c;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        if (n < N) out[n] = *s_offset + s_scan[tid] - c;
        __syncthreads();
        if (tid == 0) *s_offset += s_scan[255];
        __syncthreads();
    }
    return *s_offset;
}

__global__ __launch_bounds__(256) void chunk_table_kernel(int N, int T, const int32_t *__restrict__ cu_in,
                                                          int32_t *__restrict__ meta,
                                                          int32_t *__restrict__ cu_ws,
                                                          int32_t *__restrict__ row0,
                                                          int32_t *__restrict__ row_tok,
                                                          int32_t *__restrict__ row_len, int seg_chunks,
                                                          int32_t *__restrict__ seg_first,
                                                          int32_t *__restrict__ seg_cnt,
                                                          int32_t *__restrict__ seg_tab, int tables) {
    __shared__ int s_code;
    __shared__ int s_scan[256];
    __shared__ int s_offset;
    const int tid = threadIdx.x;
    if (tid == 0) s_code = 0;
    __syncthreads();
    for (int n = tid; n <= N; n += 256) {
        const int val = cu_in[n];
        cu_ws[n] = val;
        if (n == 0 && val != 0) atomicOr(&s_code, 1);
        if (n > 0 && cu_in[n - 1] > val) atomicOr(&s_code, 2);
        if (n == N && val != T) atomicOr(&s_code, 4);
    }
    __syncthreads();
    const int code = s_code;
    if (code) {
        if (tid == 0) {
            meta[0] = 0;
            meta[1] = (code & 1) ? 1 : ((code & 2) ? 2 : 3);
            meta[2] = 0;
        }
        return;
    }
    if (!tables) {   // the call's kernels need only the check
        if (tid == 0) {
            meta[0] = 0;
            meta[1] = 0;
            meta[2] = 0;
        }
        return;
    }
    auto chunks = [&](int n) { return (cu_in[n + 1] - cu_in[n] + C - 1) / C; };
    const int rows = block_exclusive_scan(N, chunks, row0, s_scan, &s_offset);
    int units = 0;
    if (seg_chunks > 0) {
        auto segs = [&](int n) { return max(1, (chunks(n) + seg_chunks - 1) / seg_chunks); };
        units = block_exclusive_scan(N, segs, seg_first, s_scan, &s_offset);
        for (int n = tid; n < N; n += 256) {
            const int ns = segs(n), u0 = seg_first[n];
            seg_cnt[n] = ns;
            for (int j = 0; j < ns; ++j) {
                seg_tab[2 * (u0 + j)] = n;
                seg_tab[2 * (u0 + j) + 1] = j;
            }
        }
    }
    if (tid == 0) {
        meta[0] = rows;
        meta[1] = 0;
        meta[2] = units;
    }
    for (int n = tid; n < N; n += 256) {
        const int s0 = cu_in[n], s1 = cu_in[n + 1];
        const int r = row0[n];
        for (int j = 0; j * C < s1 - s0; ++j) {
            row_tok[r + j] = s0 + j * C;
            row_len[r + j] = min(C, s1 - s0 - j * C);
        }
    }
}

// ============================================================================
// G1: one wave per (chunk row, head) item, no block barriers:
//   g = inclusive scan of log alpha, gamma_r = e^{g_r}, kappa_r = e^{g_C - g_r},
//   P = (Q K^T) o Gamma,  A = strictLower(diag(beta) (Gamma o K K^T)),
//   T = (I + A)^{-1},  M = T diag(beta).
//
// Q and K go from global memory straight into matrix-core operand registers:
// for row block b (rows 16b .. 16b + 15) lane (n, j) (n = l % 16, j = l / 16)
// holds dk indices 32p + 8j .. 32p + 8j + 7 of row 16b + n, for every k-tile
// pair p.  The product of row blocks X (first operand) and Y (second) then
// leaves lane (n, j) holding (Y X^T)[n][4j .. 4j + 3]: the "row layout" R of
// that 16 x 16 tile.  R is also the order P and M are stored in (tile t of
// a row = 256 consecutive elements, lane l owning elements 4l .. 4l + 3),
// which is the operand fragment G2 reads for them.
//
// The 64 x 64 inverse works on 16 x 16 blocks:
//   diagonal      T_aa = (I + A_aa)^{-1}: lane (n, j) solves row n of T_jj by
//                 back substitution (x (I + N) = e_n, last column first),
//                 reading N^T of its block from LDS;
//   off-diagonal  T_ab = -T_aa U_ab,  U_ab = sum_{b <= m < a} A_am T_mb, by
//                 distance a - b, on fp32 matrix cores.
// Besides R(X), tiles appear transposed, C(X): lane (n, j) holds
// X[4j .. 4j + 3][n].  One fp32 16 x 16 x 16 product turns (R(A), C(B)) into
// C(AB), and equally (C(U), R(T)) into R(TU), so T_ab is produced in R layout
// for M and, where a later U needs it, in C layout as well.
// ============================================================================

// 2^x for x <= 0 with the hardware base-2 exponential (about 1 ulp; large
// negative arguments flush to 0, never NaN).  G1 keeps g in base-2 units
// (g log2 e), so the decay masks need no extra multiply.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_neg(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS of one G1 wave, in floats: g, beta, the reciprocal row norms of Q and
// K and kappa / ||k|| for the 64 rows, then four 16 x 16 blocks (N^T of each
// diagonal block during the solve, T_aa after it).  Row pitch 20 and block pitch 324 keep the
// 16-byte row reads, the column reads and the four-block broadcast reads free
// of bank conflicts.
constexpr int kPrepBP = 20;
constexpr int kPrepBS = 16 * kPrepBP + 4;
constexpr int kPrepLds = 5 * C + 4 * kPrepBS;

// One 16 x 16 x 16 tile product of the inverse: (R(A), C(B)) -> C(AB) + acc,
// or equally (C(U), R(T)) -> R(TU) + acc, fp32 sums.  When M is stored in
// fp16 the operands are rounded to fp16 (one instruction; the rounding is
// that of the stored M); fp32 M keeps fp32 operands (four instructions).
template <typename OP>
struct InvMma;
template <>
struct InvMma<_Float16> {
    __device__ __forceinline__ static float4_t mm(const float4_t &x, const float4_t &y, float4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_convertvector(x, half4_t),
                                                    __builtin_convertvector(y, half4_t), acc, 0, 0, 0);
    }
};
template <>
struct InvMma<float> {
    __device__ __forceinline__ static float4_t mm(const float4_t &x, const float4_t &y, float4_t acc) {
        return mm16_f32(x, y, acc);
    }
};

// The UT transform and the decay-masked Q K^T of one chunk from the wave's
// Gram accumulators (R layout, the 10 lower tiles; pacc = Q K^T, gacc =
// K K^T): P = (Q K^T) o Gamma with the normalisation factors, A =
// strictLower(diag(beta)(Gamma o K K^T)), T = (I + A)^{-1} and M = T diag(beta).
// Written in fragment order (tile t at t * 256, lane l's four values at 4 l):
//   m_out = diag(kappa / ||k||) M   (the state pass's update takes
//           diag(kappa / ||k||) V' = m_out Y, and V' itself is not needed)
//   p_out = P M                     (the output's intra-chunk term P V' =
//           (P M) Y, lower triangular like P and M)
// The scratch holds, per row r of the chunk (lane r wrote them): gs = g_r
// log2 e, bs = beta_r, qn = 1 / ||q_r||, kn = 1 / ||k_r||, kh = kappa_r /
// ||k_r||, then the four 16 x 16 blocks of the diagonal inverse.  One wave, no
// block barriers.
template <typename OP>
__device__ __forceinline__ void ut_epilogue(const float4_t (&pacc)[kTriTiles], const float4_t (&gacc)[kTriTiles],
                                            float *lds, OP *p_out, OP *m_out) {
    using M = Mma<OP>;
    using MI = InvMma<OP>;
    constexpr int BP = kPrepBP, BS = kPrepBS;
    const float *gs = lds, *bs = lds + C, *qn = lds + 2 * C, *kn = lds + 3 * C, *kh = lds + 4 * C;
    float *blk = lds + 5 * C;
    const int l = lane_id(), nn = l & 15, jj = l >> 4;
    // Decay masks (g in base-2 units).  Off-diagonal tiles: row r = 16a + n, columns
    // c = 16b + 4j + i < r, one exponential shared by P and A.  Diagonal
    // tiles: the lane's positions with c <= r belong to P; the others
    // give N^T[n][c - 16a] = A[c][r] of the same block, whose decay is
    // e^{g_c - g_r}, so again one exponential per position.
    float gr[4], br[4], iqr[4], ikr[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        gr[a] = gs[16 * a + nn];
        br[a] = bs[16 * a + nn];
        iqr[a] = qn[16 * a + nn];
        ikr[a] = kn[16 * a + nn];
    }
    float4_t aR[kTriTiles];   // R(-A_ab) for a > b
    float4_t pR[kTriTiles];   // R(P_ab)
#pragma unroll
    for (int t = 0; t < kTriTiles; ++t) {
        int a, b;
        tri_decode(t, a, b);
        const float4_t gc = *reinterpret_cast<const float4_t *>(gs + 16 * b + 4 * jj);
        const float4_t kc = *reinterpret_cast<const float4_t *>(kn + 16 * b + 4 * jj);   // column factors
        float4_t pv, av;
        if (a > b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = exp2_neg(gr[a] - gc[i]) * kc[i];
                pv[i] = e * iqr[a] * pacc[t][i];
                av[i] = -br[a] * ikr[a] * e * gacc[t][i];
            }
            aR[t] = av;
        } else {
            const float4_t bc = *reinterpret_cast<const float4_t *>(bs + 16 * a + 4 * jj);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool lower = 4 * jj + i <= nn;
                const float x = gr[a] - gc[i];
                const float e = exp2_neg(lower ? x : -x) * kc[i];
                pv[i] = lower ? e * iqr[a] * pacc[t][i] : 0.f;
                av[i] = lower ? 0.f : bc[i] * ikr[a] * e * gacc[t][i];
            }
            *reinterpret_cast<float4_t *>(blk + a * BS + nn * BP + 4 * jj) = av;
            aR[t] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
        pR[t] = pv;
    }
    asm volatile("" ::: "memory");

    // Diagonal blocks: lane (n, j) computes row n of T_jj.
    diag_block_inverse<BP, BS>(blk, nn, jj);
    float4_t tR[4], tC[4];   // R(T_aa), C(T_bb)
#pragma unroll
    for (int a = 0; a < 4; ++a) tR[a] = *reinterpret_cast<const float4_t *>(blk + a * BS + nn * BP + 4 * jj);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) tC[b][i] = blk[b * BS + (4 * jj + i) * BP + nn];

    // Off-diagonal blocks by distance from the diagonal.
    const float4_t z = {0.f, 0.f, 0.f, 0.f};
    float4_t TR[kTriTiles], TC[kTriTiles];   // R(T_ab), C(T_ab)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        TR[tri_index(a, a)] = tR[a];
        TC[tri_index(a, a)] = tC[a];
    }
    // W = -U_ab (from the negated A tiles); T_ab = T_aa W in R layout and in
    // C layout (C layout feeds the later U's and the products with M below).
    float4_t W;
    W = MI::mm(aR[tri_index(1, 0)], tC[0], z);
    TR[tri_index(1, 0)] = MI::mm(W, tR[1], z);
    TC[tri_index(1, 0)] = MI::mm(tR[1], W, z);
    W = MI::mm(aR[tri_index(2, 1)], tC[1], z);
    TR[tri_index(2, 1)] = MI::mm(W, tR[2], z);
    TC[tri_index(2, 1)] = MI::mm(tR[2], W, z);
    W = MI::mm(aR[tri_index(3, 2)], tC[2], z);
    TR[tri_index(3, 2)] = MI::mm(W, tR[3], z);
    TC[tri_index(3, 2)] = MI::mm(tR[3], W, z);
    W = MI::mm(aR[tri_index(2, 1)], TC[tri_index(1, 0)], MI::mm(aR[tri_index(2, 0)], tC[0], z));
    TR[tri_index(2, 0)] = MI::mm(W, tR[2], z);
    TC[tri_index(2, 0)] = MI::mm(tR[2], W, z);
    W = MI::mm(aR[tri_index(3, 2)], TC[tri_index(2, 1)], MI::mm(aR[tri_index(3, 1)], tC[1], z));
    TR[tri_index(3, 1)] = MI::mm(W, tR[3], z);
    TC[tri_index(3, 1)] = MI::mm(tR[3], W, z);
    W = MI::mm(aR[tri_index(3, 2)], TC[tri_index(2, 0)],
               MI::mm(aR[tri_index(3, 1)], TC[tri_index(1, 0)], MI::mm(aR[tri_index(3, 0)], tC[0], z)));
    TR[tri_index(3, 0)] = MI::mm(W, tR[3], z);
    TC[tri_index(3, 0)] = MI::mm(tR[3], W, z);

    // M = T diag(beta): in C layout (lane (n, j) holds column 16 b + n) for
    // the products P M, and in R layout scaled by kappa / ||k|| per row for
    // the state pass.
    float kr[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) kr[a] = kh[16 * a + nn];
#pragma unroll
    for (int t = 0; t < kTriTiles; ++t) {
        int a, b;
        tri_decode(t, a, b);
        const float4_t bc = *reinterpret_cast<const float4_t *>(bs + 16 * b + 4 * jj);
        float4_t mv;
#pragma unroll
        for (int i = 0; i < 4; ++i) mv[i] = TR[t][i] * bc[i] * kr[a];
        *reinterpret_cast<typename M::frag *>(m_out + t * kTileElems + 4 * l) = M::cvt(mv);
        TC[t] = TC[t] * bs[16 * b + nn];
    }
    // (P M)_ab = sum over b <= m <= a of P_am M_mb: R(P_am M_mb) from
    // (C(M_mb), R(P_am)).
#pragma unroll
    for (int t = 0; t < kTriTiles; ++t) {
        int a, b;
        tri_decode(t, a, b);
        float4_t acc = z;
#pragma unroll
        for (int m = b; m <= a; ++m) acc = MI::mm(TC[tri_index(m, b)], pR[tri_index(a, m)], acc);
        *reinterpret_cast<typename M::frag *>(p_out + t * kTileElems + 4 * l) = M::cvt(acc);
    }
    asm volatile("" ::: "memory");   // the scratch is reused by the wave's next item
}

// Register passes over dk in G1: the raw Q and K registers of one pass
// stay within 128 per lane, so two waves fit on a SIMD and one computes
// while the other waits for its loads.
template <typename in_t, int DK>
struct PrepShape {
    static constexpr int KP = DK / 32;   // k-tile pairs along dk
    static constexpr int REGS_PER_PAIR = 2 * 4 * (int)sizeof(Raw8<in_t>) / 4;
    static constexpr int NPASS = KP * REGS_PER_PAIR > 128 ? KP * REGS_PER_PAIR / 128 : 1;
    static constexpr int PP = KP / NPASS;   // k-tile pairs per pass
    static_assert(PP * NPASS == KP, "dk must split evenly into passes");
    // Resident waves per SIMD the register allocation must allow: two up to
    // dk = 128 for 16-bit inputs and dk = 64 for fp32 (one wave's loads
    // overlap the other's products); the larger forms take what they need.
    static constexpr int WAVES = DK * (int)sizeof(in_t) <= 256 ? 2 : 1;
};

// Raw Q and K operand registers of one item (one pass over dk) and its
// decay inputs.
template <typename in_t, int PP>
struct PrepRegs {
    Raw8<in_t> k[4][PP], q[4][PP];
    float la, bt;
};

template <typename in_t, typename OP, int DK>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(PrepShape<in_t, DK>::WAVES))) void chunk_prep_kernel(int H, int T, int cpr, int urows, int qk_norm,
                                                        const int32_t *__restrict__ meta,
                                                        const int32_t *__restrict__ row_tok,
                                                        const int32_t *__restrict__ row_len,
                                                        const in_t *__restrict__ q,
                                                        const in_t *__restrict__ k,
                                                        const float *__restrict__ log_alpha,
                                                        const float *__restrict__ beta,
                                                        float *__restrict__ ws_g,
                                                        OP *__restrict__ ws_m,
                                                        OP *__restrict__ ws_p) {
    using M = Mma<OP>;
    using L = PrepShape<in_t, DK>;
    using MI = InvMma<OP>;
    constexpr int NPASS = L::NPASS, PP = L::PP;
    constexpr int BP = kPrepBP, BS = kPrepBS;
    __shared__ __align__(16) float lds[kPrepLds];
    float *gs = lds, *bs = lds + C, *qn = lds + 2 * C, *kn = lds + 3 * C, *kh = lds + 4 * C, *blk = lds + 5 * C;

    const int l = threadIdx.x, nn = l & 15, jj = l >> 4;
    const int rows = cpr ? urows : meta[0];
    const int64_t tok_stride = (int64_t)H * DK;

    // Issue the loads of pass s of an item (no waits).  Row indices are
    // clamped to the sequence; process() zeroes the rows past its end.
    auto load = [&](int item, int s, PrepRegs<in_t, PP> &R) {
        const int row = item / H, h = item % H;
        int tok0, len;
        row_span(row, T, cpr, row_tok, row_len, tok0, len);
        if (s == 0) {
            const int r = min(l, len - 1);
            R.la = log_alpha[(int64_t)(tok0 + r) * H + h];
            R.bt = beta[(int64_t)(tok0 + r) * H + h];
        }
        const int64_t base = ((int64_t)tok0 * H + h) * DK + 8 * jj + 32 * s * PP;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t off = base + (int64_t)min(16 * b + nn, len - 1) * tok_stride;
#pragma unroll
            for (int p = 0; p < PP; ++p) R.k[b][p].load(k + off + 32 * p);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t off = base + (int64_t)min(16 * b + nn, len - 1) * tok_stride;
#pragma unroll
            for (int p = 0; p < PP; ++p) R.q[b][p].load(q + off + 32 * p);
        }
    };

    // Everything of one item once pass 0 of its loads has been issued into R.
    auto process = [&](int item, PrepRegs<in_t, PP> &R) {
        const int row = item / H;
        int tok0, len;
        row_span(row, T, cpr, row_tok, row_len, tok0, len);
        const int64_t rh = item;   // == row * H + h

        // Rows past the end of the sequence get log alpha = 0, beta = 0 and
        // zero Q and K rows: g stays flat there and those rows are inert in
        // every product.
        auto mask_rows = [&]() {
            if (len < C) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (16 * b + nn >= len)
#pragma unroll
                        for (int p = 0; p < PP; ++p) {
                            R.k[b][p].zero();
                            R.q[b][p].zero();
                        }
            }
        };
        float la = R.la, bt = R.bt;
        if (l >= len) la = bt = 0.f;
        const float g = wave_inclusive_scan(la);
        const float g_last = __shfl(g, C - 1, 64);
        gs[l] = g * kLog2e;   // base-2 units for the decay masks
        bs[l] = bt;
        const float gam = expf(g);             // gamma_r: decay from the chunk start
        const float kap = expf(g_last - g);    // kappa_r: decay from row r to the chunk end

        // Lower-triangular tiles (a, b), b <= a, of Q K^T and K K^T in R
        // layout: first operand row block b of K, second row block a.
        float4_t pacc[kTriTiles], gacc[kTriTiles];
#pragma unroll
        for (int t = 0; t < kTriTiles; ++t) pacc[t] = gacc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
        float ssk[4] = {0.f, 0.f, 0.f, 0.f}, ssq[4] = {0.f, 0.f, 0.f, 0.f};   // row sums of squares
#pragma unroll
        for (int s = 0; s < NPASS; ++s) {
            if (s > 0) {
                __builtin_amdgcn_sched_barrier(0);
                load(item, s, R);
            }
            mask_rows();
            if (qk_norm) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int p = 0; p < PP; ++p) {
                        float f[8];
                        R.k[b][p].to_f32(f);
#pragma unroll
                        for (int e = 0; e < 8; ++e) ssk[b] += f[e] * f[e];
                        R.q[b][p].to_f32(f);
#pragma unroll
                        for (int e = 0; e < 8; ++e) ssq[b] += f[e] * f[e];
                    }
            }
#pragma unroll
            for (int t = 0; t < kTriTiles; ++t) {
                int a, b;
                tri_decode(t, a, b);
#pragma unroll
                for (int p = 0; p < PP; ++p) {
                    gram_mma(gacc[t], R.k[b][p], R.k[a][p]);
                    gram_mma(pacc[t], R.k[b][p], R.q[a][p]);
                }
            }
        }

        // L2 normalisation of the Q and K rows (when asked for) is applied as
        // row and column factors of the products: Qn Kn^T = D_q (Q K^T) D_k
        // with D = diag(1 / ||row||).  Lane (n, j) has the partial sums of
        // squares of rows 16b + n over its dk pieces; the four lanes of a row
        // add theirs.  A zero row keeps a factor of 0 (it stays zero).  The
        // factors are 1 without normalisation.  Lane l keeps row l's.
        float rq = 1.f, rk = 1.f;
        if (qk_norm) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                ssk[b] += __shfl_xor(ssk[b], 16, 64);
                ssk[b] += __shfl_xor(ssk[b], 32, 64);
                ssq[b] += __shfl_xor(ssq[b], 16, 64);
                ssq[b] += __shfl_xor(ssq[b], 32, 64);
            }
            const float sk = jj == 0 ? ssk[0] : (jj == 1 ? ssk[1] : (jj == 2 ? ssk[2] : ssk[3]));
            const float sq = jj == 0 ? ssq[0] : (jj == 1 ? ssq[1] : (jj == 2 ? ssq[2] : ssq[3]));
            rk = sk > 0.f ? rsqrtf(sk) : 0.f;
            rq = sq > 0.f ? rsqrtf(sq) : 0.f;
        }
        qn[l] = rq;
        kn[l] = rk;
        kh[l] = kap * rk;
        // Decay factors for the state pass, with the normalisation folded in:
        // gamma / ||k|| (scales K S^T in Y), kappa / ||k|| (the update), gamma
        // / ||q|| (the output), and gamma itself (the chunk's total decay).
        ws_g[rh * 4 * C + l] = gam * rk;
        ws_g[rh * 4 * C + C + l] = kap * rk;
        ws_g[rh * 4 * C + 2 * C + l] = gam * rq;
        ws_g[rh * 4 * C + 3 * C + l] = gam;
        asm volatile("" ::: "memory");

        ut_epilogue<OP>(pacc, gacc, lds, ws_p + rh * kTriTiles * kTileElems,
                                    ws_m + rh * kTriTiles * kTileElems);
    };

    // Block b takes row 8 (b / 8 / H) + b mod 8, head (b / 8) mod H: the H
    // items of a chunk row then share one XCD (workgroups go to the 8 XCDs
    // round-robin by block id, and the grid is a multiple of 8), so the
    // row's [token][head] lines of log alpha and beta are fetched into one
    // L2 rather than eight.
    const int vitems = (rows + 7) / 8 * 8 * H;
    PrepRegs<in_t, PP> R;
    for (int vb = blockIdx.x; vb < vitems; vb += gridDim.x) {
        const int slot = vb >> 3, row = slot / H * 8 + (vb & 7);
        if (row >= rows) continue;
        const int item = row * H + slot % H;
        load(item, 0, R);
        process(item, R);
    }
}

// ============================================================================
// G2: serial state pass.  Block = NW waves = 16*NW value columns of one
// (sequence, head).  Blocks of one (sequence, head) are placed on the same
// XCD (workgroups are dispatched to the 8 XCDs round-robin by block id) so
// the Q, K, M, P blocks they all read are shared through that XCD's L2.
//
// Products per chunk and wave (16 value columns v, S^T slice in sT):
//   X_K = K S^T                            (C x 16)   A: K rows,     B: sT
//   Y   = V - diag(gamma) X_K                         V read transposed
//   D   = (diag(kappa) M) Y                (C x 16)   A: diag(kappa) M, B: Y
//   O^T = (S Q^T) diag(gamma) + Y^T (P M)^T (16 x C)  A: sT / Y,     B: Q, P M rows
//   S^T = gamma_C S^T + K^T D              (dk x 16)  A: K read transposed, B: D
// (M, P and kappa here carry the q/k normalisation factors G1 folds in.)
// O is produced transposed so each lane holds four consecutive value columns
// of one token row and writes them with one vector store.
//
// Order of dk inside the state registers: tile 2p + h, lane (n, j), element
// i holds S^T[32p + 8j + 4h + i][n].  Read as a k-tile pair, lane j then
// covers dk 32p + 8j .. 32p + 8j + 7, eight consecutive values, so every
// Q or K operand fragment is one 16-byte LDS read of a row.
//
// Staging.  Q and K are loaded into registers one chunk ahead, converted to
// operand precision and written to LDS; V, M, P and the decay factors are
// copied global -> LDS by direct loads (16 bytes per lane, lane order) into
// the buffer of the next chunk while the current chunk is computed.  V rows
// have no padding; their 16-byte units are XOR-swizzled by row so the
// transposed reads do not collide in the LDS banks.  Q and K rows are padded
// by 32 bytes, which makes both the 16-byte row reads and the transposed
// reads conflict-free.  Q and K are double-buffered when LDS allows, so a
// chunk needs one barrier; otherwise a second barrier separates their
// commit from the reads.
// ============================================================================
// Waves of a state-pass block that stage inputs (the others compute): four,
// and six in an output-pass block of two compute waves, which then has eight
// waves (two per SIMD) and more loads in flight per compute unit (the
// stagers' loads are what such a block waits for).
constexpr int kStagers = 4;

template <typename in_t, typename OP, int DK, int NW, bool OUT>
struct StateSmem {
    static constexpr int NLD = (NW == 2 && OUT) ? 6 : kStagers;        // loading waves
    static constexpr int WAVES = NW + NLD;
    static constexpr int BV = 16 * NW;                                  // value columns per block
    static constexpr int QROW = DK * (int)sizeof(OP) + 32;              // bytes per Q / K row
    static constexpr int VROW = BV * (int)sizeof(in_t);                 // bytes per V row
    static constexpr int VUNITS = VROW / 16;                            // 16-byte units per V row
    static constexpr int VSWZ = VUNITS >= 8 ? 7 : VUNITS - 1;           // unit XOR mask (row bits)
    static constexpr size_t QK = (size_t)C * QROW;                      // one Q or K block
    static constexpr int NQK = OUT ? 2 : 1;                             // Q and K, or K alone
    static constexpr size_t VB = (size_t)C * VROW;
    static constexpr size_t MP = sizeof(OP) * kTriTiles * kTileElems;   // one M or P block
    static constexpr int NMP = OUT ? 2 : 1;                             // M and P, or M alone
    static constexpr size_t GB = 1024;                                  // the four decay vectors
    static constexpr size_t DMA = VB + NMP * MP + GB;                   // a chunk's copied inputs
    static constexpr int QKB = (2 * NQK * QK + 2 * DMA <= 160 * 1024) ? 2 : 1;   // Q/K buffers
    static constexpr size_t qk_off(int b) { return (size_t)b * NQK * QK; }       // Q (if any), then K
    static constexpr size_t k_rel = OUT ? QK : 0;
    static constexpr size_t dma_off(int b) { return (size_t)QKB * NQK * QK + (size_t)b * DMA; }
    static constexpr size_t m_rel = VB, p_rel = VB + MP, g_rel = VB + NMP * MP;
    static constexpr size_t in_bytes = (size_t)QKB * NQK * QK + 2 * DMA;
    // Output staging (OBUF): two buffers of a chunk's output rows for the
    // block's BV value columns (fp32 or 16-bit, OPITCH bytes per token), so
    // that the rows go to HBM as whole cache lines rather than as each
    // wave's 16-column pieces.  Used when a block holds at least two column
    // groups and the buffers fit beside the rest.
    static constexpr int OPITCH = BV * 4 + 16;
    static constexpr size_t ob_off = (in_bytes + 15) / 16 * 16;
    static constexpr bool OBUF = OUT && QKB == 2 && NW >= 2 && ob_off + 2 * (size_t)C * OPITCH <= 160 * 1024;
    static constexpr size_t ob_bytes = OBUF ? (size_t)C * OPITCH : 0;
    static constexpr size_t bytes = OBUF ? ob_off + 2 * ob_bytes : in_bytes;
    static constexpr int NV = (int)(VB / 1024), NM = (int)(MP / 1024);
    static constexpr int NMC = NM;                                        // copies of M
    static constexpr int NPC = OUT ? NM : 0;                              // copies of P
    static constexpr int NGC = 1;                                         // copies of the decay factors
    static constexpr int NDMA = NV + NMC + NPC + NGC;                     // 1 KiB wave copies per chunk
    static_assert(VB % 1024 == 0 && MP % 1024 == 0, "direct loads move whole 1 KiB wave blocks");
    static_assert(QROW % 16 == 0 && VROW % 16 == 0, "16-byte rows");
};

// Segmentation of the state pass (see the launcher): chunks per segment
// (0 = whole sequences), segments per sequence of an equal-length batch, the
// packed batch's unit tables, and the two per-unit state buffers.
struct SegArgs {
    int seg_chunks, nsegc;
    const int32_t *seg_cnt, *seg_tab;
    float *ws_end;          // per (unit, head): (DV + DK) x DK, the segment's map from zero / identity
    float *ws_sin;          // per (unit, head): DV x DK, the state entering the segment
};


// V in accumulator layout: V[R + i][c] for lane (c = c0 + n, R = row0 + 4 j),
// i < 4.  16-bit V uses one transposed read at the lane's address `a`; fp32
// V reads the four rows at the four lane addresses a[0..3].  read() returns
// the raw bits, to_f32() converts them, so the conversion (which waits for
// the read) can sit later than the read.
template <typename T>
struct VFrag;
template <>
struct VFrag<bf16_t> {
    using raw = uint2;
    __device__ __forceinline__ static raw read(const unsigned char *base, const int (&a)[4]) {
        return lds_read_tr16(base + a[0]);
    }
    __device__ __forceinline__ static float4_t to_f32(raw r) {
        return float4_t{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                        __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
    }
};
template <>
struct VFrag<_Float16> {
    using raw = uint2;
    __device__ __forceinline__ static raw read(const unsigned char *base, const int (&a)[4]) {
        return lds_read_tr16(base + a[0]);
    }
    __device__ __forceinline__ static float4_t to_f32(raw r) {
        const half4_t h = __builtin_bit_cast(half4_t, r);
        return float4_t{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    }
};
template <>
struct VFrag<float> {
    using raw = float4_t;
    __device__ __forceinline__ static raw read(const unsigned char *base, const int (&a)[4]) {
        return float4_t{*reinterpret_cast<const float *>(base + a[0]), *reinterpret_cast<const float *>(base + a[1]),
                        *reinterpret_cast<const float *>(base + a[2]), *reinterpret_cast<const float *>(base + a[3])};
    }
    __device__ __forceinline__ static float4_t to_f32(raw r) { return r; }
};

// K^T operand fragment (rows = dk, k = tokens) of one k-tile: lane (n, j)
// gets K[R + i][d(n)], i < 4.  fp16: one transposed read at `a` (bytes from
// the K block); fp32: four reads, rows QROW apart.
__device__ __forceinline__ half4_t kt_frag(const unsigned char *p, int, _Float16 *) {
    return __builtin_bit_cast(half4_t, lds_read_tr16(p));
}
__device__ __forceinline__ float4_t kt_frag(const unsigned char *p, int qrow, float *) {
    return float4_t{*reinterpret_cast<const float *>(p), *reinterpret_cast<const float *>(p + qrow),
                    *reinterpret_cast<const float *>(p + 2 * qrow), *reinterpret_cast<const float *>(p + 3 * qrow)};
}

// One 1 KiB wave copy global -> LDS: lane l's 16 bytes at g land at lds + 16 l
// (gfx950 direct load to LDS; the LDS base is wave-uniform and goes in M0).
// Written as inline assembly so the compiler does not treat every later LDS
// read as possibly depending on the copy: completion is awaited explicitly
// (s_waitcnt vmcnt before the barriers).  M0 is saved and restored around
// it, and one wait state separates the M0 write from the load.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
        : "memory");
}

template <typename in_t, typename OP, int DK, int NW, bool OUT>
__global__ __launch_bounds__((64 * StateSmem<in_t, OP, DK, NW, OUT>::WAVES)) void chunk_state_kernel(
    int NU, int H, int DV, int nvt, int odt, int T, int cpr, int32_t *__restrict__ meta,
    const int32_t *__restrict__ cu_ws, const int32_t *__restrict__ row0, SegArgs sg,
    const in_t *__restrict__ q, const in_t *__restrict__ k, const in_t *__restrict__ v,
    const float *__restrict__ ws_g, const OP *__restrict__ ws_m, const OP *__restrict__ ws_p,
    const float *init_state, float *final_state, void *__restrict__ o) {
    using M = Mma<OP>;
    using frag = typename M::frag;
    using F2 = Frag2<OP>;
    using L = StateSmem<in_t, OP, DK, NW, OUT>;
    constexpr int QROW = L::QROW, VROW = L::VROW, BV = L::BV, QKB = L::QKB;
    constexpr int NLD = L::NLD;                              // loading waves
    constexpr int NT = 64 * NLD;                             // loading threads
    constexpr int KT = DK / 16;                              // state tiles along dk
    constexpr int KP = DK / 32;                              // k-tile pairs along dk
    constexpr int QK_UNITS = C * (DK / 8);                   // 8-element pieces of Q (and K)
    // With six staging waves (waves 2..7; wave w runs on SIMD w mod 4) the
    // four on the SIMDs without a compute wave stage Q and K, and the two
    // that share a SIMD with one (waves 4, 5) issue only the direct copies,
    // so the conversions' VALU work stays off the compute waves' SIMDs.
    constexpr bool ROLES = NLD == 6 && L::QKB == 2 && OUT;   // (double-buffered Q/K: the order below)
    constexpr int QNT = ROLES ? 256 : NT;                    // threads staging Q and K
    constexpr int QK_IT = (QK_UNITS + QNT - 1) / QNT;
    constexpr int NDW = ROLES ? 2 : NLD;                     // waves issuing the direct copies
    constexpr int OPB = (int)sizeof(OP);
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;       // LDS address of smem

    if (cpr) {
        // Equal-length batch: no table pass ran, so report its row count and
        // a clean status for the host-side check here.
        if (OUT && blockIdx.x == 0 && threadIdx.x == 0) {
            meta[0] = (int)((int64_t)NU / H / (sg.seg_chunks ? sg.nsegc : 1)) * ((T + C - 1) / C);
            meta[1] = 0;
        }
    } else if (meta[1] != 0) {
        return;
    }
    // Block -> (unit, value tile).  A unit is one (sequence, segment, head);
    // the blocks of a unit sit on one XCD (workgroups go to the 8 XCDs
    // round-robin by block id) so they share its Q, K, M, P lines in L2.
    const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
    const int unit = (slot / nvt) * 8 + xcd, vt = slot % nvt;
    if (unit >= NU) return;
    const int useg = unit / H, h = unit % H;
    int n, seg, nseg;   // sequence, segment within it, its segment count
    if (sg.seg_chunks == 0) {
        n = useg, seg = 0, nseg = 1;
    } else if (cpr) {
        n = useg / sg.nsegc, seg = useg - n * sg.nsegc, nseg = sg.nsegc;
    } else {
        if (useg >= meta[2]) return;
        n = sg.seg_tab[2 * useg], seg = sg.seg_tab[2 * useg + 1], nseg = sg.seg_cnt[n];
    }
    // The transition of a sequence's last segment is never needed.
    if (!OUT && seg == nseg - 1) return;
    // Columns of the running state: the value columns, and for a transition
    // pass over a segment after the first, DK more that start as the
    // identity and see zero values (they carry the segment's map F).
    const int DVA = (!OUT && seg > 0) ? DV + DK : DV;
    const int vb = vt * BV;                 // first value column of the block
    if (vb >= DVA) return;
    const int chain = n * H + h;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, nn = l & 15, jj = l >> 4;
    // Waves 0..NW-1 compute: wave w holds 16 value columns (column group
    // cg = w); the L::NLD waves after them stage the next chunk's inputs
    // into LDS.
    const bool stager = w >= NW;
    const int sw = w - NW;                          // stager wave index
    const bool qk_role = !ROLES || (sw & 2) == 0;   // stages Q and K (with ROLES: stager waves 0, 1, 4, 5)
    // thread index among the Q/K stagers, and wave index among the copying waves
    const int stid = ROLES ? ((sw >> 2) * 2 + (sw & 1)) * 64 + l : tid - 64 * NW;
    const int dsw = ROLES ? (sw & 1) : sw;
    const int cg = w;
    const int v0 = vb + cg * 16;            // first value column of a compute wave
    const bool active = !stager && v0 < DVA;
    const bool ident = v0 >= DV;            // a column of F (transition pass only)
    // The chunks this block runs: all of the sequence's, or one segment.
    int tok0 = cpr ? n * T : cu_ws[n];
    int len_seq = cpr ? T : cu_ws[n + 1] - tok0;
    int r0 = cpr ? n * cpr : row0[n];
    if (sg.seg_chunks) {
        const int cb = seg * sg.seg_chunks;
        tok0 += cb * C;
        r0 += cb;
        len_seq = max(0, min(len_seq - cb * C, sg.seg_chunks * C));
    }
    const int nchunks = (len_seq + C - 1) / C;

    // ---- per-lane LDS byte offsets ----
    const int frag_lane = nn * QROW + 8 * jj * OPB;                 // Q / K row fragments
    int kt_lane;                                                    // K^T fragments
    if constexpr (OPB == 2)
        kt_lane = (4 * jj + (nn >> 2)) * QROW + 16 * (nn & 3);
    else
        kt_lane = 4 * jj * QROW + 4 * (8 * (nn >> 2) + (nn & 3));
    int v_lane[4];                                                  // V in accumulator layout
    if constexpr (sizeof(in_t) == 2) {
        const int row = 4 * jj + (nn >> 2), unit = 2 * cg + ((nn & 3) >> 1);
        v_lane[0] = row * VROW + 16 * (unit ^ (row & L::VSWZ)) + 8 * (nn & 1);
        v_lane[1] = v_lane[2] = v_lane[3] = v_lane[0];
    } else {
        const int unit = 4 * cg + (nn >> 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * jj + i;
            v_lane[i] = row * VROW + 16 * (unit ^ (row & L::VSWZ)) + 4 * (nn & 3);
        }
    }
    const int tile_lane = 4 * l;                                    // M / P tiles (elements)

    // S^T tiles in the dk order described above.  The state entering the
    // block's chunks: the caller's initial state (whole sequences, or the
    // transition pass over a first segment), the segment's incoming state
    // from the combine pass (output pass over segments), or zero / identity
    // (transition pass over a later segment).
    float4_t sT[KT];
    const float *s_in = nullptr;
    int64_t s_in_row = 0;   // element offset of the lane's state row
    if (OUT && sg.seg_chunks) {
        s_in = sg.ws_sin;
        s_in_row = ((int64_t)unit * DV + v0 + nn) * DK;
    } else if (seg == 0) {
        s_in = init_state;
        s_in_row = ((int64_t)chain * DV + v0 + nn) * DK;
    }
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int off = 32 * (t >> 1) + 4 * (t & 1);
        if (active && s_in && !ident) {
            sT[t] = *reinterpret_cast<const float4_t *>(s_in + s_in_row + 8 * jj + off);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)   // S^T[d][c] = [d == c - DV] on identity columns
                sT[t][i] = (active && ident && 8 * jj + off + i == v0 + nn - DV) ? 1.f : 0.f;
        }
    }

    // ---- Q / K register prefetch ----
    // Two register sets: the loads for one chunk are issued before the other
    // set is converted and committed, so they have a whole chunk to land.
    // Loads use the chunk's first row as a uniform base plus 32-bit per-lane
    // offsets; in a partial chunk the rows past the end re-read the last
    // valid row and are zeroed when committed to LDS.
    struct QKRegs {
        Raw8<in_t> q[QK_IT], k[QK_IT];
    };
    QKRegs RA, RB;
    const int rowq = H * DK;   // element stride between tokens
    int offq[QK_IT];
#pragma unroll
    for (int it = 0; it < QK_IT; ++it) {
        const int u = (stid + it * QNT) % QK_UNITS;
        offq[it] = (u / (DK / 8)) * rowq + (u % (DK / 8)) * 8;
    }
    auto prefetch_qk = [&](int ci, QKRegs &R) {
        const int64_t tb = (int64_t)(tok0 + ci * C) * H + h;
        const int last = min(C, len_seq - ci * C) - 1;
        const in_t *qc = q + tb * DK;
        const in_t *kc = k + tb * DK;
        if (last == C - 1) {
#pragma unroll
            for (int it = 0; it < QK_IT; ++it) {
                if constexpr (OUT) R.q[it].load(qc + offq[it]);
                R.k[it].load(kc + offq[it]);
            }
        } else {
#pragma unroll
            for (int it = 0; it < QK_IT; ++it) {
                const int u = (stid + it * QNT) % QK_UNITS;
                const int off = min(u / (DK / 8), last) * rowq + (u % (DK / 8)) * 8;
                if constexpr (OUT) R.q[it].load(qc + off);
                R.k[it].load(kc + off);
            }
        }
    };
    auto commit_qk = [&](int b, int len, QKRegs &R) {
        OP *Qb = reinterpret_cast<OP *>(smem + L::qk_off(b));
        OP *Kb = reinterpret_cast<OP *>(smem + L::qk_off(b) + L::k_rel);
#pragma unroll
        for (int it = 0; it < QK_IT; ++it) {
            const int u = stid + it * QNT;
            if (u >= QK_UNITS) continue;
            const int r = u / (DK / 8), c8 = (u % (DK / 8)) * 8;
            if (len < C && r >= len) {
                if constexpr (OUT) R.q[it].zero();
                R.k[it].zero();
            }
            frag lo, hi;
            if constexpr (OUT) {
                to_op(R.q[it], lo, hi);
                store_row8(Qb + r * (QROW / OPB) + c8, lo, hi);
            }
            to_op(R.k[it], lo, hi);
            store_row8(Kb + r * (QROW / OPB) + c8, lo, hi);
        }
    };
    // ---- direct global -> LDS copies of V, M, P and the decay factors ----
    // Copy ii of a chunk (stager wave sw issues ii = sw, sw + NLD, ...) fills LDS bytes
    // [1024 ii, 1024 ii + 1024) of the chunk's buffer: V blocks first, then
    // M, P (output pass only) and the 4C decay factors.  Per-lane source
    // offsets do not depend on the chunk and are computed once.  Rows past the
    // end of a partial chunk re-read the last valid row: M and P are exactly
    // zero in those rows and columns, so they stay inert.  Columns past DV
    // (inactive waves, or the F columns of a transition pass, which use zero
    // values) read column 0 and are not used.
    constexpr int KD = (L::NDMA + NDW - 1) / NDW;
    int dsrc[KD];   // V: elements from the chunk's first row; M, P, g: bytes
#pragma unroll
    for (int kx = 0; kx < KD; ++kx) {
        const int ii = dsw + NDW * kx;
        if (ii < L::NV) {
            const int byte = ii * 1024 + 16 * l;
            const int row = byte / VROW, unit = (byte % VROW) / 16;
            int col = vb + (unit ^ (row & L::VSWZ)) * (16 / (int)sizeof(in_t));
            if (col >= DV) col = 0;
            dsrc[kx] = row * H * DV + col;
        } else if (ii < L::NV + L::NMC + L::NPC) {
            dsrc[kx] = ((ii - L::NV) % L::NM) * 1024 + 16 * l;
        } else {
            dsrc[kx] = 16 * l;
        }
    }
    auto dma = [&](int ci, int b) {
        const int64_t rh = (int64_t)(r0 + ci) * H + h;
        const int len = min(C, len_seq - ci * C);
        const uint32_t base = lds0 + (uint32_t)L::dma_off(b);
        const in_t *vc = v + ((int64_t)(tok0 + ci * C) * H + h) * DV;
        const unsigned char *mc = reinterpret_cast<const unsigned char *>(ws_m + rh * kTriTiles * kTileElems);
        const unsigned char *pc = reinterpret_cast<const unsigned char *>(ws_p + rh * kTriTiles * kTileElems);
        const unsigned char *gc = reinterpret_cast<const unsigned char *>(ws_g + rh * 4 * C);
#pragma unroll
        for (int kx = 0; kx < KD; ++kx) {
            const int ii = dsw + NDW * kx;
            if (ii >= L::NDMA) break;
            if (ii < L::NV) {
                int off = dsrc[kx];
                if (len < C) {
                    const int row = (ii * 1024 + 16 * l) / VROW;
                    if (row >= len) off -= (row - (len - 1)) * H * DV;
                }
                dma16(vc + off, base + (uint32_t)(ii * 1024));
            } else if (ii < L::NV + L::NMC) {
                dma16(mc + dsrc[kx], base + (uint32_t)(L::m_rel + (ii - L::NV) * 1024));
            } else if (ii < L::NV + L::NMC + L::NPC) {
                dma16(pc + dsrc[kx], base + (uint32_t)(L::p_rel + (ii - L::NV - L::NMC) * 1024));
            } else {
                dma16(gc + dsrc[kx], base + (uint32_t)L::g_rel);
            }
        }
    };

    // Finish the initial-state loads here, and re-issue the state registers
    // as produced after that wait, so no wait inside the loop is attached to
    // these loads.
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int t = 0; t < KT; ++t) asm volatile("" : "+v"(sT[t]));

    // Output tiles (fp32, and rounded to 16 bits and packed) and store addresses.
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    float4_t oq[4] = {};
    u32x2_t oh[4] = {};
    uint64_t oa[4] = {};
    const int osize = odt == DT_FP32 ? 4 : 2;
    // The lane's output address in the block's first chunk; a chunk and a
    // row tile further on are uniform byte offsets.
    const uint64_t o_lane = reinterpret_cast<uint64_t>(o) +
                            (uint64_t)((((int64_t)tok0 * H + h) * DV + v0 + 4 * jj + (int64_t)nn * H * DV) * osize);
    const int64_t o_chunk = (int64_t)C * H * DV * osize, o_tile = (int64_t)16 * H * DV * osize;
    // Stores of NR row tiles (row tile rt0 + r from oq[r]).  The output type
    // and a partial chunk are decided once for all of them, so the stores
    // issue as straight-line code.
    auto store_rows = [&](int ci, int len, auto NRc, int rt0) {
        constexpr int NR = decltype(NRc)::value;
#pragma unroll
        for (int r = 0; r < NR; ++r) oa[r] = o_lane + (uint64_t)(ci * o_chunk + (rt0 + r) * o_tile);
        if (odt == DT_FP32) {
            if (len == C) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    __builtin_nontemporal_store(oq[r], reinterpret_cast<__attribute__((address_space(1))) float4_t *>(oa[r]));
            } else {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    if (16 * (rt0 + r) + nn < len)
                        __builtin_nontemporal_store(oq[r], reinterpret_cast<__attribute__((address_space(1))) float4_t *>(oa[r]));
            }
            return;
        }
        if (odt == DT_BF16) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                oh[r] = u32x2_t{pack_bf16x2(oq[r][0], oq[r][1]), pack_bf16x2(oq[r][2], oq[r][3])};
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                oh[r] = __builtin_bit_cast(u32x2_t, half4_t{(_Float16)oq[r][0], (_Float16)oq[r][1],
                                                            (_Float16)oq[r][2], (_Float16)oq[r][3]});
        }
        if (len == C) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                __builtin_nontemporal_store(oh[r], reinterpret_cast<__attribute__((address_space(1))) u32x2_t *>(oa[r]));
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (16 * (rt0 + r) + nn < len)
                    __builtin_nontemporal_store(oh[r], reinterpret_cast<__attribute__((address_space(1))) u32x2_t *>(oa[r]));
        }
    };
    auto store_o = [&](int ci, int len) { store_rows(ci, len, std::integral_constant<int, 4>{}, 0); };

    // OBUF: chunk ci's output tiles go to staging buffer ci & 1 (each lane
    // its four rows' 4 values, fp32 or rounded to 16 bits); after the next
    // block barrier every compute wave stores an equal share of the chunk's
    // rows, each store instruction covering whole rows of the block's
    // columns (OB_N per wave: the rows' bytes are BV * osize, 16 per lane).
    // (only in blocks whose column groups are all within DV)
    const bool obuf = L::OBUF && vb + BV <= DV;
    const uint64_t o_blk = reinterpret_cast<uint64_t>(o) + (uint64_t)((((int64_t)tok0 * H + h) * DV + vb) * osize);
    const int64_t o_row = (int64_t)H * DV * osize;
    auto stage_o = [&](int ci) {
        unsigned char *ob = smem + L::ob_off + (size_t)(ci & 1) * L::ob_bytes;
        if (odt == DT_FP32) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                *reinterpret_cast<float4_t *>(ob + (16 * rt + nn) * L::OPITCH + 4 * (16 * cg + 4 * jj)) = oq[rt];
            return;
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            oh[rt] = odt == DT_BF16 ? u32x2_t{pack_bf16x2(oq[rt][0], oq[rt][1]), pack_bf16x2(oq[rt][2], oq[rt][3])}
                                    : __builtin_bit_cast(u32x2_t, half4_t{(_Float16)oq[rt][0], (_Float16)oq[rt][1],
                                                                         (_Float16)oq[rt][2], (_Float16)oq[rt][3]});
            *reinterpret_cast<u32x2_t *>(ob + (16 * rt + nn) * L::OPITCH + 2 * (16 * cg + 4 * jj)) = oh[rt];
        }
    };
    // Rows of staged chunk cs (a whole chunk: only a sequence's last chunk
    // can be partial, and that one is stored directly); flusher fi of NW
    // stores its share.
    auto flush_o = [&](int cs, int fi) {
        const unsigned char *ob = smem + L::ob_off + (size_t)(cs & 1) * L::ob_bytes;
        const uint64_t oc = o_blk + (uint64_t)(cs * o_chunk);
        if (odt == DT_FP32) {
            constexpr int LPR = BV * 4 / 16, TPI = 64 / LPR, PER = LPR / NW;   // lanes per row, rows per store
            const int tr = l / LPR, cb = 16 * (l % LPR);
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int tok = (fi * PER + j) * TPI + tr;
                const float4_t d = *reinterpret_cast<const float4_t *>(ob + tok * L::OPITCH + cb);
                __builtin_nontemporal_store(d, reinterpret_cast<__attribute__((address_space(1))) float4_t *>(
                                                   oc + (uint64_t)(tok * o_row + cb)));
            }
        } else {
            constexpr int LPR = BV * 2 / 16, TPI = 64 / LPR, PER = LPR / NW;
            const int tr = l / LPR, cb = 16 * (l % LPR);
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int tok = (fi * PER + j) * TPI + tr;
                const float4_t d = *reinterpret_cast<const float4_t *>(ob + tok * L::OPITCH + cb);
                __builtin_nontemporal_store(d, reinterpret_cast<__attribute__((address_space(1))) float4_t *>(
                                                   oc + (uint64_t)(tok * o_row + cb)));
            }
        }
    };


    // The two roles run separate loops with the same barriers: one per chunk
    // (two with a single Q/K buffer).  Before a barrier a stager waits for
    // its direct loads, Q/K register loads (in the output pass all but the
    // newest chunk's) and LDS writes; a compute wave
    // waits only for its LDS reads, never for its output stores, which drain
    // in the background.  After the barrier the staged chunk is visible and
    // every wave is done with chunk ci-1's buffers.  The barriers are written
    // out (rather than __syncthreads) so that no wait for outstanding global
    // stores is attached to them.
    //
    // Stager step ci (QKB == 2): issue chunk ci+2's Q and K loads into `nxt`
    // and copy chunk ci+1's V, M, P and decay factors, then commit chunk
    // ci+1's Q and K from `cur` (the order differs between the passes, see
    // below).  With a single Q/K buffer (QKB == 1) chunk ci is committed
    // between the two barriers.
    auto stage = [&](int ci, QKRegs &cur, QKRegs &nxt) {
        const int b = ci & 1;
        if constexpr (QKB == 2 && OUT)   // all but this wave's newest Q/K prefetch (below)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * QK_IT) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if constexpr (QKB == 1) {
            if (ci > 0) commit_qk(0, min(C, len_seq - ci * C), cur);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        if constexpr (QKB == 2 && OUT) {
            // Output pass: chunk ci+1's copies first, then chunk ci+2's Q and K,
            // then chunk ci+1's Q and K committed from `cur` (the compiler's
            // wait for `cur` also covers the copies, which are older than the
            // new Q/K loads).  The next barrier waits for everything but those
            // Q/K loads, so they have two chunk steps to land.
            // (near the end the last chunk is loaded again: the register
            // sets are then written on every path, which keeps them in place)
            if (ci + 1 < nchunks) dma(ci + 1, b ^ 1);
            prefetch_qk(min(ci + 2, nchunks - 1), nxt);
            if (ci + 1 < nchunks) commit_qk(b ^ 1, min(C, len_seq - (ci + 1) * C), cur);
        } else if constexpr (QKB == 2) {
            // Transition pass: chunk ci+2's K loads and chunk ci+1's copies,
            // then chunk ci+1's K committed from `cur` (complete since the
            // barrier's wait; `touch` keeps the compiler from waiting again
            // behind the new loads).
#pragma unroll
            for (int it = 0; it < QK_IT; ++it) cur.k[it].touch();
            prefetch_qk(min(ci + 2, nchunks - 1), nxt);
            if (ci + 1 < nchunks) {
                dma(ci + 1, b ^ 1);
                commit_qk(b ^ 1, min(C, len_seq - (ci + 1) * C), cur);
            }
        } else {
#pragma unroll
            for (int it = 0; it < QK_IT; ++it) {
                if constexpr (OUT) cur.q[it].touch();
                cur.k[it].touch();
            }
            prefetch_qk(min(ci + 1, nchunks - 1), nxt);
            if (ci + 1 < nchunks) dma(ci + 1, b ^ 1);
        }
    };
    // Register budgets of a compute step (see its phases): K (and Q) row
    // fragments, registers per fragment pair, registers for read-ahead
    // fragments, and how many K and Q fragments are held at once.
    constexpr int NX = 4 * KP;
    constexpr int FR = 4 * OPB / 2;
    constexpr int RBR = KT > 8 ? 32 : 64;
    constexpr int WX = NX < RBR / FR ? NX : RBR / FR;
    constexpr int WQ = NX / 2 < RBR / 2 / FR ? NX / 2 : RBR / 2 / FR;
    constexpr int NQ1 = NX / 2;                     // Q S^T items before the update
    // Compute step ci.
    auto compute = [&](auto ci) {   // (generic: instantiated only where called)
        const int len = min(C, len_seq - ci * C);
        const int b = ci & 1;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if constexpr (QKB == 1) asm volatile("s_barrier" ::: "memory");
        if (!active) return;

        const unsigned char *Qb = smem + L::qk_off(QKB == 2 ? b : 0);   // (output pass only)
        const unsigned char *Kb = Qb + L::k_rel;
        const unsigned char *Db = smem + L::dma_off(b);
        const OP *Ms = reinterpret_cast<const OP *>(Db + L::m_rel);
        const OP *Ps = reinterpret_cast<const OP *>(Db + L::p_rel);
        // decay factors (G1): gamma / ||k||, kappa / ||k|| (folded into M here,
        // not read), gamma / ||q||, gamma
        const float *gam_s = reinterpret_cast<const float *>(Db + L::g_rel);
        const float *gao_s = gam_s + 2 * C;

        // The chunk is software-pipelined: each phase issues the LDS reads of
        // a later phase before its own products, and the phases are pinned
        // in order (scheduling barriers), so read latency hides behind
        // matrix-core and vector work.  Row-fragment item i of K or Q is
        // (k-tile pair i / 4, row tile i % 4); consecutive products of a phase
        // go to different accumulators.
        auto rd_row = [&](const unsigned char *blk, int i) {
            return row_frag2(reinterpret_cast<const OP *>(blk + 16 * (i % 4) * QROW + frag_lane) + 32 * (i / 4));
        };
        // D = (diag(kappa) M) Y and Y^T (P M)^T use the lower-triangular tiles of M and P as
        // k-tile pairs: row tile mt takes pair 0 (tiles (mt,0),(mt,1)) and,
        // for mt >= 2, pair 1 (tiles (mt,2),(mt,3)); absent tiles are zero.
        auto tri_pair = [&](const OP *T, int mt, int p) {
            const int k0 = 2 * p, k1 = 2 * p + 1;
            const frag lo = k0 <= mt ? lds_frag(T + tri_index(mt, k0) * kTileElems + tile_lane) : M::zero();
            const frag hi = k1 <= mt ? lds_frag(T + tri_index(mt, k1) * kTileElems + tile_lane) : M::zero();
            return F2::make(lo, hi);
        };
        // pair j of the six: (mt, p) = (0,0) (1,0) (2,0) (3,0) (2,1) (3,1), so
        // products into one accumulator are never back to back
        constexpr int PMT[6] = {0, 1, 2, 3, 2, 3}, PP[6] = {0, 0, 0, 0, 1, 1};
        // K^T fragments of state tile t = 2p + hs (dk 32p + 8j + 4hs + i) for
        // token pair tp: K columns 32p + 8 (n/4) + 4hs + n%4.
        auto rd_kt = [&](int t, int tp) {
            const int p = t >> 1, hs = t & 1;
            const unsigned char *kt = Kb + kt_lane + OPB * (32 * p + 4 * hs) + 32 * tp * QROW;
            return F2::make(kt_frag(kt, QROW, (OP *)nullptr), kt_frag(kt + 16 * QROW, QROW, (OP *)nullptr));
        };

        // -- phase 0: K fragments, V, gamma; S as an operand; decay of S.
        // LDS reads complete in order, so gamma_C is read first: the decay
        // waits for it alone, not for the fragments behind it. --
        const float gC = gam_s[4 * C - 1];
        F2 kf[WX];
#pragma unroll
        for (int i = 0; i < WX; ++i) kf[i] = rd_row(Kb, i);
        typename VFrag<in_t>::raw vraw[4];
        float4_t gm[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            vraw[mt] = VFrag<in_t>::read(Db + 16 * mt * VROW, v_lane);
            gm[mt] = *reinterpret_cast<const float4_t *>(gam_s + 16 * mt + 4 * jj);
        }
        F2 sB[KP];            // B of K S^T and A of S Q^T
#pragma unroll
        for (int p = 0; p < KP; ++p) sB[p] = F2::cvt(sT[2 * p], sT[2 * p + 1]);
#pragma unroll
        for (int t = 0; t < KT; ++t) sT[t] *= gC;   // the update adds K^T D later
        __builtin_amdgcn_sched_barrier(0);

        // -- phase 1: X_K = K S^T; reads of M and the first Q fragments --
        float4_t x[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) x[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            mma2(x[i % 4], kf[i % WX], sB[i / 4]);
            if (i + WX < NX) kf[i % WX] = rd_row(Kb, i + WX);
        }
        F2 mpair[6];
#pragma unroll
        for (int jx = 0; jx < 6; ++jx) mpair[jx] = tri_pair(Ms, PMT[jx], PP[jx]);
        F2 qf[WQ];
        if constexpr (OUT) {
#pragma unroll
            for (int i = 0; i < WQ; ++i) qf[i] = rd_row(Qb, i);
        }
        __builtin_amdgcn_sched_barrier(0);

        // -- phase 2: Y = V - diag(gamma) X_K as B operand --
        F2 yB[2];
        {
            float4_t y[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)   // the F columns of a transition pass see v = 0
                y[mt] = (ident ? float4_t{0.f, 0.f, 0.f, 0.f} : VFrag<in_t>::to_f32(vraw[mt])) - gm[mt] * x[mt];
            yB[0] = F2::cvt(y[0], y[1]);
            yB[1] = F2::cvt(y[2], y[3]);
        }
        __builtin_amdgcn_sched_barrier(0);

        // -- phase 3: D = diag(kappa) V' = (diag(kappa) M) Y; the first K^T fragments --
        float4_t Dk[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Dk[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jx = 0; jx < 6; ++jx) mma2(Dk[PMT[jx]], mpair[jx], yB[PP[jx]]);
        constexpr int NT1 = KT < RBR / 4 / FR ? KT : RBR / 4 / FR;   // K^T tiles read ahead
        F2 ka[KT][2];
#pragma unroll
        for (int t = 0; t < NT1; ++t) {
            ka[t][0] = rd_kt(t, 0);
            ka[t][1] = rd_kt(t, 1);
        }
        __builtin_amdgcn_sched_barrier(0);

        // -- phase 4: the first half of Q S^T (independent of the chain) --
        float4_t qs[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) qs[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (OUT) {
#pragma unroll
            for (int i = 0; i < NQ1; ++i) {
                mma2(qs[i % 4], sB[i / 4], qf[i % WQ]);
                if (i + WQ < NX) qf[i % WQ] = rd_row(Qb, i + WQ);
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        // -- phase 5: the operand form of D --
        F2 dB[2];
        dB[0] = F2::cvt(Dk[0], Dk[1]);
        dB[1] = F2::cvt(Dk[2], Dk[3]);
        __builtin_amdgcn_sched_barrier(0);

        // The previous chunk's rows (staged before this chunk's barrier) go
        // out here, after the stagers have issued this step's loads.
        if constexpr (L::OBUF && !ROLES) {   // (with the staging roles the copying waves flush)
            if (obuf && ci > 0) flush_o(ci - 1, cg);
        }
        // -- phase 6: state update, K^T fragments read NT1 tiles ahead; the
        // two products of a tile are NT1 apart, not back to back --
#pragma unroll
        for (int t = 0; t < KT + NT1; ++t) {
            if (t < KT) {
                if (t + NT1 < KT) {
                    ka[t + NT1][0] = rd_kt(t + NT1, 0);
                    ka[t + NT1][1] = rd_kt(t + NT1, 1);
                }
                mma2(sT[t], ka[t][0], dB[0]);
            }
            if (t >= NT1) mma2(sT[t - NT1], ka[t - NT1][1], dB[1]);
        }
        if constexpr (!OUT) return;   // a transition pass stops at the update
        F2 ppair[6];
#pragma unroll
        for (int jx = 0; jx < 6; ++jx) ppair[jx] = tri_pair(Ps, PMT[jx], PP[jx]);
        float g1[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) g1[rt] = gao_s[16 * rt + nn];
        __builtin_amdgcn_sched_barrier(0);

        // -- phase 7: rest of Q S^T, then Y^T (P M)^T into a separate sum --
#pragma unroll
        for (int i = NQ1; i < NX; ++i) {
            mma2(qs[i % 4], sB[i / 4], qf[i % WQ]);
            if (i + WQ < NX) qf[i % WQ] = rd_row(Qb, i + WQ);
        }
        float4_t pv[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) pv[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jx = 0; jx < 6; ++jx) mma2(pv[PMT[jx]], yB[PP[jx]], ppair[jx]);
        // O^T = (S Q^T) diag(gamma) + Y^T (P M)^T
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) oq[rt] = qs[rt] * g1[rt] + pv[rt];
        if constexpr (L::OBUF) {
            if (obuf && ci + 1 < nchunks) {
                stage_o(ci);
                return;
            }
        }
        store_o(ci, len);
    };

    if constexpr (ROLES) {
        if (stager && qk_role) {
            // Q/K staging: chunk ci+2's loads, then chunk ci+1 committed; the
            // barrier leaves the newest chunk's loads outstanding.
            if (nchunks > 0) {
                prefetch_qk(0, RA);
                commit_qk(0, min(C, len_seq), RA);
                if (nchunks > 1) prefetch_qk(1, RB);
            }
            auto step_qk = [&](int ci, QKRegs &cur, QKRegs &nxt) {
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * QK_IT) : "memory");
                prefetch_qk(min(ci + 2, nchunks - 1), nxt);
                if (ci + 1 < nchunks) commit_qk((ci + 1) & 1, min(C, len_seq - (ci + 1) * C), cur);
            };
            int ci = 0;
            for (; ci + 1 < nchunks; ci += 2) {
                step_qk(ci, RB, RA);
                step_qk(ci + 1, RA, RB);
            }
            if (ci < nchunks) step_qk(ci, RB, RA);
            return;
        }
        if (stager) {   // direct copies of V, M, P and the decay factors, one chunk ahead,
                        // and the output rows the compute waves staged in the previous step
            if (nchunks > 0) dma(0, 0);
            for (int ci = 0; ci < nchunks; ++ci) {
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                if (ci + 1 < nchunks) dma(ci + 1, (ci + 1) & 1);
                if constexpr (L::OBUF) {
                    if (obuf && ci > 0) flush_o(ci - 1, dsw);
                }
            }
            return;
        }
    }
    if (stager) {
        if (nchunks > 0) {
            prefetch_qk(0, RA);
            dma(0, 0);
            commit_qk(0, min(C, len_seq), RA);
            if (QKB == 2 && nchunks > 1) prefetch_qk(1, RB);
        }
        // Register sets alternate: with QKB == 2, chunk ci+1 sits in RB for
        // even ci and in RA for odd ci; with QKB == 1, chunk ci does.  Steps
        // run in pairs so both sets are written on every path.
        int ci = 0;
        for (; ci + 1 < nchunks; ci += 2) {
            if constexpr (QKB == 2) {
                stage(ci, RB, RA);
                stage(ci + 1, RA, RB);
            } else {
                stage(ci, RA, RB);
                stage(ci + 1, RB, RA);
            }
        }
        if (ci < nchunks) {
            if constexpr (QKB == 2)
                stage(ci, RB, RA);
            else
                stage(ci, RA, RB);
        }
        return;
    }
    for (int ci = 0; ci < nchunks; ++ci) compute(ci);

    // The state leaving the block's chunks: the sequence's final state (output
    // pass over its last segment), or the segment's map (transition pass).
    float *s_out = nullptr;
    int64_t s_out_row = 0;
    if (!OUT) {
        s_out = sg.ws_end;
        s_out_row = ((int64_t)unit * (DV + DK) + v0 + nn) * DK;
    } else if (seg == nseg - 1 && final_state) {
        s_out = final_state;
        s_out_row = ((int64_t)chain * DV + v0 + nn) * DK;
    }
    if (active && s_out) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
            *reinterpret_cast<float4_t *>(s_out + s_out_row + 8 * jj + 32 * (t >> 1) + 4 * (t & 1)) = sT[t];
    }
}

// ============================================================================
// Combine pass of a segmented state pass.  Segment s of a sequence maps the
// state entering it to the state leaving it as S -> S F_s + G_s (every chunk
// step is affine in S: S_next = S (gamma_C I - K^T diag(gamma) M^T diag(kappa) K)
// + V^T M^T diag(kappa) K, and a segment composes its chunks' maps).  The
// transition pass left [G_s; F_s] in ws_end (G_s from a zero state, F_s from
// the identity through the same chunks with zero values); for the first
// segment it left the true leaving state.  Per (sequence, head, 16 state
// rows) this pass walks the segments in order and writes the state entering
// each one to ws_sin:
//   S_in(0) = initial state (or 0),  S_in(1) = ws_end(0),
//   S_in(s + 1) = S_in(s) F_s + G_s.
// fp32 throughout.  Thread t owns row 16 rt + t / 16 and DK / 16 consecutive
// columns.  For each product the block's 16 rows of S sit in LDS, and F goes
// through LDS in slabs of SLAB rows (16-byte loads into registers, issued one
// slab ahead), so each thread's sums read LDS only.
// ============================================================================
template <int DK>
struct CombineSmem {
    static constexpr int SLAB = DK <= 64 ? DK : 8192 / DK;   // F rows per slab (at most 32 KiB)
    static constexpr int LD = SLAB * DK / 4 / 256;            // 16-byte loads per thread per slab
    static_assert(LD * 256 * 4 == SLAB * DK, "a slab is whole 16-byte loads of all 256 threads");
};

template <int DK>
__global__ __launch_bounds__(256) void chunk_combine_kernel(int NSEQ, int H, int DV, int cpr, const int32_t *meta,
                                                            SegArgs sg, const int32_t *__restrict__ seg_first,
                                                            const float *init_state) {
    constexpr int CPT = DK / 16;   // columns per thread
    using L = CombineSmem<DK>;
    constexpr int SLAB = L::SLAB;
    __shared__ __align__(16) float rows[16][DK + 4];
    __shared__ __align__(16) float fs[SLAB][DK];
    const int nrt = DV / 16;
    const int rt = blockIdx.x % nrt, nh = blockIdx.x / nrt;
    const int n = nh / H, h = nh % H;
    if (n >= NSEQ) return;
    if (!cpr && meta[1] != 0) return;   // malformed cu_seqlens: nothing is written
    const int nseg = cpr ? sg.nsegc : sg.seg_cnt[n];
    const int u0 = cpr ? n * sg.nsegc : seg_first[n];
    const int t = threadIdx.x, r = 16 * rt + t / 16, c0 = (t % 16) * CPT;
    auto unit = [&](int s) { return (int64_t)(u0 + s) * H + h; };
    float S[CPT];
    const float *src = init_state ? init_state + ((int64_t)nh * DV + r) * DK + c0 : nullptr;
#pragma unroll
    for (int j = 0; j < CPT; ++j) S[j] = src ? src[j] : 0.f;
    auto put = [&](int s) {
        float *dst = sg.ws_sin + (unit(s) * DV + r) * DK + c0;
        if constexpr (CPT % 4 == 0) {
#pragma unroll
            for (int j = 0; j < CPT; j += 4)
                *reinterpret_cast<float4_t *>(dst + j) = float4_t{S[j], S[j + 1], S[j + 2], S[j + 3]};
        } else {
#pragma unroll
            for (int j = 0; j < CPT; ++j) dst[j] = S[j];
        }
    };
    put(0);
    if (nseg < 2) return;
    {
        const float *e = sg.ws_end + (unit(0) * (DV + DK) + r) * DK + c0;
#pragma unroll
        for (int j = 0; j < CPT; ++j) S[j] = e[j];
    }
    put(1);
    // The products S_in(s + 1) = S_in(s) F_s + G_s for s = 1 .. nseg - 2, as
    // one sequence of slab steps; each step issues the next step's F slab
    // and G rows (indices clamped at the last step, so no branch surrounds a
    // load) before it computes, so the walk waits on L2 / HBM only once.
    constexpr int NSL = DK / SLAB;
    const int nsteps = (nseg - 2) * NSL;
    if (nsteps <= 0) return;
    auto slab = [&](int step) {
        const int s = 1 + step / NSL;
        return sg.ws_end + unit(s) * (DV + DK) * DK + (int64_t)(DV + step % NSL * SLAB) * DK;
    };
    auto grow = [&](int step) { return sg.ws_end + (unit(1 + step / NSL) * (DV + DK) + r) * DK + c0; };
    float4_t ld[L::LD];
    float gn[CPT];
    auto load = [&](int step) {
        const float *F = slab(step), *G = grow(step);
#pragma unroll
        for (int i = 0; i < L::LD; ++i) ld[i] = *reinterpret_cast<const float4_t *>(F + 4 * (t + 256 * i));
#pragma unroll
        for (int j = 0; j < CPT; ++j) gn[j] = G[j];
    };
    load(0);
#pragma unroll 1
    for (int step = 0; step < nsteps; ++step) {
        const int sl = step % NSL;
        __syncthreads();   // the previous step's reads of `fs` and `rows` are done
        if (sl == 0) {     // a new product: S_in(s) to `rows`, the sum starts from G_s
#pragma unroll
            for (int j = 0; j < CPT; ++j) rows[t / 16][c0 + j] = S[j];
#pragma unroll
            for (int j = 0; j < CPT; ++j) S[j] = gn[j];
        }
#pragma unroll
        for (int i = 0; i < L::LD; ++i) *reinterpret_cast<float4_t *>(&fs[0][0] + 4 * (t + 256 * i)) = ld[i];
        load(min(step + 1, nsteps - 1));
        __syncthreads();
        const int e0 = sl * SLAB;
#pragma unroll 2
        for (int e = 0; e < SLAB; e += 4) {
            const float4_t a = *reinterpret_cast<const float4_t *>(&rows[t / 16][e0 + e]);
#pragma unroll
            for (int ee = 0; ee < 4; ++ee) {
                float f[CPT];
                if constexpr (CPT % 4 == 0) {
#pragma unroll
                    for (int j = 0; j < CPT; j += 4) {
                        const float4_t x = *reinterpret_cast<const float4_t *>(&fs[e + ee][c0 + j]);
                        f[j] = x[0], f[j + 1] = x[1], f[j + 2] = x[2], f[j + 3] = x[3];
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < CPT; ++j) f[j] = fs[e + ee][c0 + j];
                }
#pragma unroll
                for (int j = 0; j < CPT; ++j) S[j] = fmaf(a[ee], f[j], S[j]);
            }
        }
        if (sl == NSL - 1) put(2 + step / NSL);
    }
}

// ============================================================================
// Host side: workspace layout and launches.
// ============================================================================
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segmented state pass.  Without it the state pass runs one chain of chunks
// per (sequence, head) and value tile, so a batch with few (sequence, head)
// pairs leaves most of the GPU idle while it walks its long chains.  Cutting
// each sequence into segments of `seg` chunks and running
//   (a) a transition pass per segment but the last (the state pass without
//       outputs, from a zero state with DK extra columns that start as the
//       identity: it leaves the segment's affine map [G; F]),
//   (b) a combine pass that walks the segments' maps to each segment's
//       incoming state, and
//   (c) the output pass per segment from that state,
// turns one chain of n chunks into two of `seg` (plus the walk).  It pays one
// more pass over K, V and M for all but the last segments, so it is used only
// when the value columns of all chains together are too few to fill the GPU:
// the segments then multiply them to about 16K columns (1024 waves of 16).
// GDN_SEG_CHUNKS overrides the choice (0 disables), for tests and tuning.
int32_t chunk_seg_chunks(int32_t B, int32_t T, int32_t N, bool packed, int32_t H, int32_t dv) {
    const char *env = getenv("GDN_SEG_CHUNKS");
    if (env && *env) {
        const int x = atoi(env);
        if (x >= 0) return x;
    }
    const int64_t rows = packed ? (T + C - 1) / C : (int64_t)B * ((T + C - 1) / C);
    if (N <= 0 || rows <= 0) return 0;
    const int64_t cols = (int64_t)N * H * dv;
    if (cols >= 8192) return 0;
    const int64_t nseg = std::min<int64_t>(16, 16384 / cols);
    const int64_t avg = (rows + N - 1) / N;             // chunks per sequence, on average
    const int64_t seg = std::max<int64_t>(8, (avg + nseg - 1) / nseg);
    return seg >= avg ? 0 : (int32_t)seg;
}

ChunkWorkspace chunk_workspace_layout(int32_t B, int32_t T, int32_t N, bool packed, int32_t H,
                                      int32_t in_dtype, int32_t dk, int32_t dv) {
    ChunkWorkspace w{};
    const int64_t per_row = (T + C - 1) / C;
    w.max_rows = packed ? per_row + N : (int64_t)B * per_row;
    w.seg_chunks = chunk_seg_chunks(B, T, N, packed, H, dv);
    if (w.seg_chunks > 0)
        w.max_units = packed ? (w.max_rows + w.seg_chunks - 1) / w.seg_chunks + N
                             : (int64_t)B * ((per_row + w.seg_chunks - 1) / w.seg_chunks);
    const size_t op = in_dtype == DT_FP32 ? 4 : 2;
    size_t off = 0;
    w.off_meta = off;   off = align256(off + 8 * sizeof(int32_t));
    w.off_cu = off;     off = align256(off + sizeof(int32_t) * (size_t)(N + 1));
    w.off_row0 = off;   off = align256(off + sizeof(int32_t) * (size_t)N);
    w.off_rowtok = off; off = align256(off + sizeof(int32_t) * (size_t)w.max_rows);
    w.off_rowlen = off; off = align256(off + sizeof(int32_t) * (size_t)w.max_rows);
    w.off_g = off;      off = align256(off + sizeof(float) * (size_t)w.max_rows * H * 4 * C);
    w.off_m = off;      off = align256(off + op * (size_t)w.max_rows * H * kTriTiles * kTileElems);
    w.off_p = off;      off = align256(off + op * (size_t)w.max_rows * H * kTriTiles * kTileElems);
    if (w.seg_chunks > 0) {
        const size_t units = (size_t)w.max_units;
        w.off_segfirst = off; off = align256(off + sizeof(int32_t) * (size_t)N);
        w.off_segcnt = off;   off = align256(off + sizeof(int32_t) * (size_t)N);
        w.off_segtab = off;   off = align256(off + sizeof(int32_t) * 2 * units);
        w.off_end = off;      off = align256(off + sizeof(float) * units * H * (size_t)(dv + dk) * dk);
        w.off_sin = off;      off = align256(off + sizeof(float) * units * H * (size_t)dv * dk);
    }
    w.total = off;
    return w;
}

// Compute waves per state-pass block (16 value columns each; the block also
// has StateSmem::NLD staging waves).  A chunk's latency does not shrink with more
// compute waves per block, so the block count is what matters: the fewest
// waves (at least 2) whose blocks still fit on the GPU in one round; 4 when
// no choice does.  GDN_STATE_WAVES (1, 2 or 4) overrides, for experiments.
// Compute units of the current device (cached after the first query).
static int cu_count() {
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

// cols: value columns per unit; units: (sequence or segment, head) units.
static int state_waves_per_block(int cols, int64_t units, const char *env_name) {
    const int cus = cu_count();
    const int tiles = (cols + 15) / 16;
    const int64_t slots = ((units + 7) / 8) * 8;
    int nw = 4;
    for (int c = 2; c <= 4; c *= 2)
        if (slots * ((tiles + c - 1) / c) <= cus) {
            nw = c;
            break;
        }
    if (tiles < nw) nw = tiles >= 2 ? 2 : 1;
    const char *env = getenv(env_name);
    if (env) {
        const int x = atoi(env);
        if (x == 1 || x == 2 || x == 4) nw = x;
    }
    return nw;
}

template <typename K>
static hipError_t allow_smem(K kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// ============================================================================
// G6: calls with few tokens per sequence (appending to resident states) on
// the matrix cores.  Each (sequence, head) runs the chunk algorithm with
// chunks of 16 tokens: per chunk the 16 x 16 matrices g, Gamma,
// A = strictLower(diag(beta)(Gamma o K K^T)), T = (I + A)^{-1},
// M = T diag(beta), P = (Q K^T) o Gamma, and
//   X_K = K S^T,  Y = V - diag(gamma) X_K,  V' = M Y,
//   O   = diag(gamma) Q S^T + P V',  S^T <- gamma_C S^T + K^T (kappa o V').
// One block per (sequence, head), one wave per 16-column value slice (up to
// kSmallMaxWaves; a wider state takes several blocks per head): a
// wave holds its slice of S^T (dk x 16 fp32, in matrix-core accumulators)
// through the sequence's chunks, so the state is read and written once.
// What does not depend on the slice is done once per chunk and shared
// through LDS: all threads stage the chunk's K and Q rows as fp16 operands
// (L2-normalised first when asked for), wave 0 scans the gates, and after a
// barrier wave 0 forms G, Q K^T, A, T, M and P while every wave forms its
// X_K and S Q^T; after a second barrier every wave finishes its slice.  The
// shared buffers alternate by chunk parity, so a chunk needs no third
// barrier before the next one overwrites them.  16-bit inputs, dk <= 128.
// ============================================================================
constexpr int kSmallC = 16;          // tokens per chunk
constexpr int kSmallMaxWaves = 16;   // value slices (waves) per block

template <int DK>
struct SmallSmem {
    static constexpr int KROW = DK * 2 + 16;                        // bytes per staged K / Q row (fp16)
    static constexpr int NTP = 20;                                  // floats per N^T row
    static constexpr size_t KQ = (size_t)kSmallC * KROW;
    // one chunk's shared operands (two sets, by chunk parity): K, Q, M in
    // the A-operand layout and P in the B-operand layout (four fp16 per
    // lane), gamma, kappa, g log2 e, beta per token and gamma_C
    static constexpr size_t K_REL = 0, Q_REL = KQ, M_REL = 2 * KQ, P_REL = M_REL + 512, VEC_REL = P_REL + 512;
    static constexpr size_t BUF = VEC_REL + (4 * kSmallC + 4) * 4;
    static constexpr size_t NT_OFF = 2 * BUF;                       // wave 0's N^T (and its T row)
    static constexpr size_t bytes = NT_OFF + (size_t)kSmallC * NTP * 4;
    static_assert(KQ % 16 == 0 && BUF % 16 == 0, "16-byte aligned regions");
};

__device__ __forceinline__ float4_t mma16(half4_t a, half4_t b, float4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ half4_t to_half4(float4_t x) { return __builtin_convertvector(x, half4_t); }

// Inclusive prefix sum over each row of 16 lanes (DPP row shifts; lanes
// shifted in from outside the row read 0).
__device__ __forceinline__ float row16_scan(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
    return x;
}

// Sum over aligned groups of RL lanes (RL = 4, 8 or 16) by DPP moves: swaps
// within quads, then the mirrored lane of the half row and of the row.
template <int RL>
__device__ __forceinline__ float group_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    if constexpr (RL >= 8)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));   // half-row mirror
    if constexpr (RL >= 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));   // row mirror
    return x;
}

template <typename in_t, typename out_t, int DK, bool INIT>
__global__ __launch_bounds__(64 * kSmallMaxWaves) void chunk_small_kernel(
    int N, int H, int DV, int T, int ng, int qk_norm, const int32_t *__restrict__ cu, int32_t *__restrict__ meta,
    const in_t *__restrict__ q, const in_t *__restrict__ k, const in_t *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta, const float *init_state,
    float *final_state, out_t *__restrict__ o) {
    using L = SmallSmem<DK>;
    using F2 = Frag2<_Float16>;
    constexpr int KROW = L::KROW, KT = DK / 16, KP = DK / 32;
    constexpr int RL = DK / 8;          // staging lanes per K / Q row (8 elements each)
    constexpr int PIECES = 4 * DK;      // 8-element pieces of the chunk's K and Q
    extern __shared__ __align__(16) unsigned char smem[];
    if (cu) {
        if (meta[1] != 0) return;   // cu_seqlens rejected by the table pass: write nothing
    } else if (blockIdx.x == 0 && threadIdx.x == 0) {
        meta[0] = N * ((T + kChunk - 1) / kChunk);
        meta[1] = 0;
    }
    // Block -> (sequence, head, first slice group); a block takes slice
    // groups g, g + ng, ... of nwv slices each.
    const int nwv = (int)(blockDim.x >> 6);
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int nh = blockIdx.x / ng, g0 = blockIdx.x % ng, n = nh / H, h = nh % H;
    const int tb = cu ? cu[n] : n * T, te = cu ? cu[n + 1] : (n + 1) * T;
    const int ns = DV / 16;
    float *NT = reinterpret_cast<float *>(smem + L::NT_OFF);
    int par = 0;   // buffer parity, carried across slice groups

    for (int s0 = g0 * nwv; s0 < ns; s0 += ng * nwv) {
        const bool has = s0 + w < ns;   // this wave has a slice in the group
        const int v0 = 16 * (s0 + w);
        // S^T slice: tile 2p + hs, lane (n, j), element i = S^T[32p + 8j + 4hs + i][v0 + n].
        // Its loads go out in the first chunk after the chunk's K and Q loads,
        // so the staging, the gate scan and wave 0's matrices proceed while
        // they are in flight (loads complete in issue order); only the
        // products with S wait for them.
        float4_t sT[KT];
        // (No branch around the loads, which would make the compiler wait for
        // them at the join: a wave without a slice reads the last slice and
        // never uses it.)
        auto load_state = [&]() {
            if constexpr (INIT) {
                const int l = threadIdx.x & 63, nn = l & 15, jj = l >> 4;
                const float *src = init_state + ((int64_t)nh * DV + (has ? v0 : DV - 16) + nn) * DK + 8 * jj;
#pragma unroll
                for (int t = 0; t < KT; ++t)
                    sT[t] = *reinterpret_cast<const float4_t *>(src + 32 * (t >> 1) + 4 * (t & 1));
            } else {
#pragma unroll
                for (int t = 0; t < KT; ++t) sT[t] = float4_t{0.f, 0.f, 0.f, 0.f};
            }
        };
        // One chunk; the first (FIRST, peeled: no branch around the state
        // loads) issues the state loads behind its K and Q loads.
        auto chunk = [&](int t0, auto FIRST) {
            const int nt = min(kSmallC, te - t0);
            // Lane-dependent values are formed anew in every chunk (the lane
            // index is opaque to the compiler here), not hoisted out of the
            // loop and held in registers across it.
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int l = tid & 63, nn = l & 15, jj = l >> 4;
            unsigned char *buf = smem + par * L::BUF;
            unsigned char *Kb = buf + L::K_REL, *Qb = buf + L::Q_REL;
            float *gam = reinterpret_cast<float *>(buf + L::VEC_REL), *kap = gam + kSmallC,
                  *gl2 = gam + 2 * kSmallC, *bv = gam + 3 * kSmallC, *gCp = gam + 4 * kSmallC;
            const int64_t th = (int64_t)t0 * H + h;

            // ---- phase A: loads.  Every load is unconditional, with indices
            // clamped to the chunk (and to the last slice for a wave without
            // one): a branch around a load makes the compiler wait for it where
            // the paths join.  Values past the end are replaced where used. ----
            const float la_in = log_alpha[th + (int64_t)min(nn, nt - 1) * H];   // (used by wave 0)
            const float bt_in = beta[th + (int64_t)min(nn, nt - 1) * H];
            in_t vr[4];
            {
                const in_t *vp = v + th * DV + (has ? v0 : DV - 16) + nn;
#pragma unroll
                for (int i = 0; i < 4; ++i) vr[i] = vp[(int64_t)min(4 * jj + i, nt - 1) * H * DV];
            }
            // K and Q rows as fp16 operands, in 8-element pieces p = tid,
            // tid + 64 nwv, ...  Rows past the end (copies of the last row)
            // need no zeroing: their beta is 0, so their rows of A and T are
            // e_n, their rows of Y and V' are 0 and they add nothing to the
            // state; their outputs are not stored.
            auto piece_src = [&](int p) {
                const int mat = p / (2 * DK), rem = p - mat * 2 * DK, r = rem / RL, c8 = rem - r * RL;
                return (mat ? q : k) + (th + (int64_t)min(r, nt - 1) * H) * DK + 8 * c8;
            };
            auto piece_store = [&](int p, const Raw8<in_t> &raw) {
                const int mat = p / (2 * DK), rem = p - mat * 2 * DK, r = rem / RL, c8 = rem - r * RL;
                float f[8];
                raw.to_f32(f);
                float sc = 1.f;
                if (qk_norm) {
                    float ss = 0.f;
#pragma unroll
                    for (int u = 0; u < 8; ++u) ss += f[u] * f[u];
                    ss = group_sum<RL>(ss);
                    sc = ss > 0.f ? rsqrtf(ss) : 0.f;
                }
                half8_t hv;
#pragma unroll
                for (int u = 0; u < 8; ++u) hv[u] = (_Float16)(f[u] * sc);
                *reinterpret_cast<half8_t *>((mat ? Qb : Kb) + r * KROW + 16 * c8) = hv;
            };
            {
                Raw8<in_t> raw0;
                raw0.load(piece_src(min(tid, PIECES - 1)));
                if constexpr (decltype(FIRST)::value) {   // behind the first K/Q loads (order pinned)
                    __builtin_amdgcn_sched_barrier(0);
                    load_state();
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (tid < PIECES) piece_store(tid, raw0);   // (wave-uniform: PIECES is a multiple of 64)
            }
            for (int p = tid + 64 * nwv; p < PIECES; p += 64 * nwv) {
                Raw8<in_t> raw;
                raw.load(piece_src(p));
                piece_store(p, raw);
            }
            if (w == 0) {   // gates: token n of the chunk in every row of 16 lanes
                const float bt = nn < nt ? bt_in : 0.f;
                const float g = row16_scan(nn < nt ? la_in : 0.f);
                const float g_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), 15));
                if (jj == 0) {
                    gam[nn] = expf(g);
                    kap[nn] = expf(g_last - g);
                    gl2[nn] = g * kLog2e;
                    bv[nn] = bt;
                    if (nn == 0) gCp[0] = expf(g_last);
                }
            }
            __syncthreads();

            // ---- phase B: products of every slice with S; wave 0 also forms
            // the chunk's shared matrices (lane (n, j) holds rows 4j .. 4j + 3,
            // column n of each product) ----
            F2 kf[KP], qf[KP];
#pragma unroll
            for (int p = 0; p < KP; ++p) {
                kf[p] = row_frag2(reinterpret_cast<const _Float16 *>(Kb + nn * KROW + 16 * jj + 64 * p));
                qf[p] = row_frag2(reinterpret_cast<const _Float16 *>(Qb + nn * KROW + 16 * jj + 64 * p));
            }
            float4_t X = {0.f, 0.f, 0.f, 0.f}, QS = X;
            if (has) {
#pragma unroll
                for (int p = 0; p < KP; ++p) {
                    const F2 sB = F2::cvt(sT[2 * p], sT[2 * p + 1]);
                    mma2(X, kf[p], sB);    // X_K[4j + i][v0 + n]
                    mma2(QS, sB, qf[p]);   // (S Q^T)[v0 + 4j + i][n]
                }
            }
            if (w == 0) {
                float4_t G = {0.f, 0.f, 0.f, 0.f}, PK = G;
#pragma unroll
                for (int p = 0; p < KP; ++p) {
                    mma2(G, kf[p], kf[p]);    // k_{4j+i} . k_n (symmetric)
                    mma2(PK, kf[p], qf[p]);   // k_{4j+i} . q_n = (Q K^T)[n][4j + i]
                }
                const float gn = gl2[nn], bn = bv[nn];
                const float4_t gc = *reinterpret_cast<const float4_t *>(gl2 + 4 * jj);
                float4_t Pr;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * jj + i;
                    const float e = c <= nn ? exp2_neg(gn - gc[i]) : 0.f;
                    Pr[i] = e * PK[i];
                    NT[c * L::NTP + nn] = c < nn ? bn * e * G[i] : 0.f;   // N^T[c][n] = A[n][c]
                }
                __builtin_amdgcn_wave_barrier();
                // row n of T = (I + A)^{-1}: x (I + A) = e_n, c = 15 .. 0 (row c
                // of N^T read as float4 broadcasts)
                float x[16];
#pragma unroll
                for (int c = 15; c >= 0; --c) {
                    float acc = 0.f;
#pragma unroll
                    for (int q4 = (c + 1) / 4; q4 < 4; ++q4) {
                        const float4_t r = *reinterpret_cast<const float4_t *>(NT + c * L::NTP + 4 * q4);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (4 * q4 + i > c) acc -= x[4 * q4 + i] * r[i];
                    }
                    x[c] = c == nn ? 1.f : acc;
                }
                // the row goes through LDS (over N^T, whose reads are done) so
                // that lane (n, j) can take its four entries 4j .. 4j + 3
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<float4_t *>(NT + nn * L::NTP + 4 * q4) =
                        float4_t{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
                __builtin_amdgcn_wave_barrier();
                const float4_t bc = *reinterpret_cast<const float4_t *>(bv + 4 * jj);
                const float4_t Mr = *reinterpret_cast<const float4_t *>(NT + nn * L::NTP + 4 * jj) * bc;   // M = T diag(beta)
                *reinterpret_cast<half4_t *>(buf + L::M_REL + 8 * l) = to_half4(Mr);
                *reinterpret_cast<half4_t *>(buf + L::P_REL + 8 * l) = to_half4(Pr);
            }
            __syncthreads();

            // ---- phase C: the slice's V', output rows and state update ----
            if (has) {
                const half4_t Mh = *reinterpret_cast<const half4_t *>(buf + L::M_REL + 8 * l);
                const half4_t Ph = *reinterpret_cast<const half4_t *>(buf + L::P_REL + 8 * l);
                const float4_t gm = *reinterpret_cast<const float4_t *>(gam + 4 * jj);
                float4_t y;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = 4 * jj + i < nt ? to_f32(vr[i]) - gm[i] * X[i] : 0.f;
                const float4_t Vp = mma16(Mh, to_half4(y), float4_t{0.f, 0.f, 0.f, 0.f});   // V' = M Y
                // O^T = (S Q^T) diag(gamma) + V'^T P^T: lane (n, j) holds O[token n][v0 + 4j + i]
                const float4_t pv = mma16(to_half4(Vp), Ph, float4_t{0.f, 0.f, 0.f, 0.f});
                const float4_t oo = QS * gam[nn] + pv;
                if (nn < nt) {
                    out_t *dst = o + (th + (int64_t)nn * H) * DV + v0 + 4 * jj;
                    if constexpr (sizeof(out_t) == 4) {
                        *reinterpret_cast<float4_t *>(dst) = oo;
                    } else if constexpr (std::is_same<out_t, bf16_t>::value) {
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(oo[0], oo[1]), pack_bf16x2(oo[2], oo[3]));
                    } else {
                        *reinterpret_cast<half4_t *>(dst) = to_half4(oo);
                    }
                }
                // S^T <- gamma_C S^T + K^T (kappa o V')
                const float gC = gCp[0];
                const float4_t kp = *reinterpret_cast<const float4_t *>(kap + 4 * jj);
                const half4_t dh = to_half4(kp * Vp);
                const unsigned char *kt = Kb + (4 * jj + (nn >> 2)) * KROW + 16 * (nn & 3);   // transposed K reads
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    const half4_t a = __builtin_bit_cast(half4_t, lds_read_tr16(kt + 2 * (32 * (t >> 1) + 4 * (t & 1))));
                    sT[t] = mma16(a, dh, sT[t] * gC);
                }
            }
            par ^= 1;
        };
        if (tb < te) {
            chunk(tb, std::true_type{});
            for (int t0 = tb + kSmallC; t0 < te; t0 += kSmallC) chunk(t0, std::false_type{});
        } else {   // no chunk: the state passes through
            load_state();
        }
        if (has && final_state) {
            const int l = threadIdx.x & 63, nn = l & 15, jj = l >> 4;
            float *dst = final_state + ((int64_t)nh * DV + v0 + nn) * DK + 8 * jj;
#pragma unroll
            for (int t = 0; t < KT; ++t)
                *reinterpret_cast<float4_t *>(dst + 32 * (t >> 1) + 4 * (t & 1)) = sT[t];
        }
    }
}

// Waves (value slices) per G6 block; GDN_SMALL_WAVES overrides, for experiments.
static int small_waves(const ChunkArgs &a) {
    const int ns = a.dv / 16;
    int waves = min(ns, kSmallMaxWaves);
    const char *env = getenv("GDN_SMALL_WAVES");
    if (env && atoi(env) >= 1 && atoi(env) <= kSmallMaxWaves) waves = min(ns, atoi(env));
    return waves;
}

template <typename in_t, typename out_t>
static hipError_t launch_small_out(const ChunkArgs &a, int32_t *meta, hipStream_t st) {
    const int ns = a.dv / 16, waves = small_waves(a);
    const int ng = (ns + waves - 1) / waves;   // blocks per (sequence, head)
    const dim3 grid((unsigned)((int64_t)a.N * a.H * ng)), block(64 * waves);
    auto *q = static_cast<const in_t *>(a.q);
    auto *k = static_cast<const in_t *>(a.k);
    auto *v = static_cast<const in_t *>(a.v);
    auto *o = static_cast<out_t *>(a.o);
    const int qn = (a.flags & kFlagQkL2Norm) ? 1 : 0;
    ProfScope prof("gdn_chunk_small", st);
    auto go = [&](auto kern, size_t lds) {
        kern<<<grid, block, lds, st>>>(a.N, a.H, a.dv, a.T, ng, qn, a.cu_seqlens, meta, q, k, v, a.log_alpha, a.beta,
                                       a.init_state, a.final_state, o);
    };
    const bool init = a.init_state != nullptr;
    switch (a.dk) {
    case 32:
        init ? go(chunk_small_kernel<in_t, out_t, 32, true>, SmallSmem<32>::bytes)
             : go(chunk_small_kernel<in_t, out_t, 32, false>, SmallSmem<32>::bytes);
        break;
    case 64:
        init ? go(chunk_small_kernel<in_t, out_t, 64, true>, SmallSmem<64>::bytes)
             : go(chunk_small_kernel<in_t, out_t, 64, false>, SmallSmem<64>::bytes);
        break;
    case 128:
        init ? go(chunk_small_kernel<in_t, out_t, 128, true>, SmallSmem<128>::bytes)
             : go(chunk_small_kernel<in_t, out_t, 128, false>, SmallSmem<128>::bytes);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
template <typename in_t>
static hipError_t launch_small_in(const ChunkArgs &a, int32_t *meta, hipStream_t st) {
    switch (a.out_dtype) {
    case DT_FP32: return launch_small_out<in_t, float>(a, meta, st);
    case DT_BF16: return launch_small_out<in_t, bf16_t>(a, meta, st);
    case DT_FP16: return launch_small_out<in_t, _Float16>(a, meta, st);
    }
    return hipErrorInvalidValue;
}
// G6 takes 16-bit inputs with dk <= 128; GDN_SMALL_CHUNKS=0 sends every
// short call to the token-serial kernel (G5) instead.
static bool use_chunk_small(const ChunkArgs &a) {
    if (a.in_dtype == DT_FP32 || a.dk > 128) return false;
    const char *env = getenv("GDN_SMALL_CHUNKS");
    return !(env && *env && atoi(env) == 0);
}
static hipError_t launch_chunk_small(const ChunkArgs &a, int32_t *meta, hipStream_t st) {
    if ((int64_t)a.N * a.H == 0) return hipSuccess;
    return a.in_dtype == DT_BF16 ? launch_small_in<bf16_t>(a, meta, st) : launch_small_in<_Float16>(a, meta, st);
}

// Chunk rows per sequence of an equal-length batch (at least 1, so that an
// empty batch still reads as equal-length), 0 for a packed one.
static int uniform_cpr(const ChunkArgs &a) { return a.cu_seqlens ? 0 : (a.T + C - 1) / C + (a.T == 0); }

template <typename in_t, typename OP, int DK, int NW, bool OUT>
static hipError_t launch_state(const ChunkArgs &a, const ChunkWorkspace &w, const SegArgs &sg, int64_t NU,
                               hipStream_t st) {
    using L = StateSmem<in_t, OP, DK, NW, OUT>;
    auto kern = chunk_state_kernel<in_t, OP, DK, NW, OUT>;
    hipError_t e = allow_smem(kern, L::bytes);
    if (e != hipSuccess) return e;
    char *ws = static_cast<char *>(a.workspace);
    const int cols = OUT ? a.dv : a.dv + a.dk;
    const int nvt = ((cols + 15) / 16 + NW - 1) / NW;
    const int64_t blocks = ((NU + 7) / 8) * 8 * nvt;
    ProfScope prof(OUT ? "gdn_chunk_state" : "gdn_chunk_transition", st);
    kern<<<dim3((unsigned)blocks), dim3(64 * L::WAVES), L::bytes, st>>>(
        (int)NU, a.H, a.dv, nvt, a.out_dtype, a.T, uniform_cpr(a), reinterpret_cast<int32_t *>(ws + w.off_meta),
        reinterpret_cast<const int32_t *>(ws + w.off_cu), reinterpret_cast<const int32_t *>(ws + w.off_row0), sg,
        static_cast<const in_t *>(a.q), static_cast<const in_t *>(a.k), static_cast<const in_t *>(a.v),
        reinterpret_cast<const float *>(ws + w.off_g), reinterpret_cast<const OP *>(ws + w.off_m),
        reinterpret_cast<const OP *>(ws + w.off_p), a.init_state, a.final_state, a.o);
    return hipGetLastError();
}

template <typename in_t, typename OP, int DK, bool OUT>
static hipError_t launch_state_nw(const ChunkArgs &a, const ChunkWorkspace &w, const SegArgs &sg, int64_t NU,
                                  hipStream_t st) {
    const int cols = OUT ? a.dv : a.dv + a.dk;
    const int nw = state_waves_per_block(cols, NU, OUT ? "GDN_STATE_WAVES" : "GDN_TRANSITION_WAVES");
    switch (nw) {
    case 4: return launch_state<in_t, OP, DK, 4, OUT>(a, w, sg, NU, st);
    case 2: return launch_state<in_t, OP, DK, 2, OUT>(a, w, sg, NU, st);
    default:
        if constexpr (OUT) return launch_state<in_t, OP, DK, 1, OUT>(a, w, sg, NU, st);
        return launch_state<in_t, OP, DK, 2, OUT>(a, w, sg, NU, st);
    }
}

template <typename in_t, typename OP, int DK>
static hipError_t launch_dk(const ChunkArgs &a, const ChunkWorkspace &w, hipStream_t st) {
    char *ws = static_cast<char *>(a.workspace);
    if (w.max_rows > 0) {   // no tokens at all: only the state pass runs (final = initial)
        ProfScope prof("gdn_chunk_prep", st);
        // One wave per (row, head) item, rows padded to a multiple of 8 (the
        // kernel's XCD placement); very large batches loop.
        const int64_t items = (w.max_rows + 7) / 8 * 8 * a.H;
        const int64_t grid = items < (1 << 22) ? items : (1 << 22);
        chunk_prep_kernel<in_t, OP, DK><<<dim3((unsigned)grid), dim3(64), 0, st>>>(
            a.H, a.T, uniform_cpr(a), (int)(uniform_cpr(a) ? w.max_rows : 0), (a.flags & kFlagQkL2Norm) ? 1 : 0,
            reinterpret_cast<const int32_t *>(ws + w.off_meta),
            reinterpret_cast<const int32_t *>(ws + w.off_rowtok),
            reinterpret_cast<const int32_t *>(ws + w.off_rowlen), static_cast<const in_t *>(a.q),
            static_cast<const in_t *>(a.k), a.log_alpha, a.beta, reinterpret_cast<float *>(ws + w.off_g),
            reinterpret_cast<OP *>(ws + w.off_m), reinterpret_cast<OP *>(ws + w.off_p));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    SegArgs sg{};
    if (w.seg_chunks == 0) return launch_state_nw<in_t, OP, DK, true>(a, w, sg, (int64_t)a.N * a.H, st);

    const int cpr = uniform_cpr(a);
    sg.seg_chunks = w.seg_chunks;
    sg.nsegc = cpr ? (cpr + w.seg_chunks - 1) / w.seg_chunks : 0;
    sg.seg_cnt = reinterpret_cast<const int32_t *>(ws + w.off_segcnt);
    sg.seg_tab = reinterpret_cast<const int32_t *>(ws + w.off_segtab);
    sg.ws_end = reinterpret_cast<float *>(ws + w.off_end);
    sg.ws_sin = reinterpret_cast<float *>(ws + w.off_sin);
    const int64_t NU = w.max_units * a.H;
    hipError_t e = launch_state_nw<in_t, OP, DK, false>(a, w, sg, NU, st);
    if (e != hipSuccess) return e;
    {
        ProfScope prof("gdn_chunk_combine", st);
        const int64_t blocks = (int64_t)a.N * a.H * (a.dv / 16);
        chunk_combine_kernel<DK><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
            a.N, a.H, a.dv, cpr, reinterpret_cast<const int32_t *>(ws + w.off_meta), sg,
            reinterpret_cast<const int32_t *>(ws + w.off_segfirst), a.init_state);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_state_nw<in_t, OP, DK, true>(a, w, sg, NU, st);
}

template <typename in_t, typename OP>
static hipError_t launch_typed(const ChunkArgs &a, const ChunkWorkspace &w, hipStream_t st) {
    switch (a.dk) {
    case 32: return launch_dk<in_t, OP, 32>(a, w, st);
    case 64: return launch_dk<in_t, OP, 64>(a, w, st);
    case 128: return launch_dk<in_t, OP, 128>(a, w, st);
    case 256:
        if constexpr (sizeof(OP) == 2) return launch_dk<in_t, OP, 256>(a, w, st);
        return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_table(int32_t N, int32_t T, const int32_t *cu_seqlens, int32_t *meta, int32_t *cu_ws,
                              int32_t *row0, int32_t *row_tok, int32_t *row_len, int32_t seg_chunks,
                              int32_t *seg_first, int32_t *seg_cnt, int32_t *seg_tab, hipStream_t st,
                              bool tables) {
    ProfScope prof("gdn_chunk_table", st);
    chunk_table_kernel<<<1, 256, 0, st>>>(N, T, cu_seqlens, meta, cu_ws, row0, row_tok, row_len, seg_chunks,
                                          seg_first, seg_cnt, seg_tab, tables ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t st) {
    const bool packed = a.cu_seqlens != nullptr;
    const ChunkWorkspace w = chunk_workspace_layout(a.B, a.T, a.N, packed, a.H, a.in_dtype, a.dk, a.dv);
    char *ws = static_cast<char *>(a.workspace);
    const bool short_call = (int64_t)a.B * a.T <= (int64_t)kShortAvg * a.N;
    if (packed) {
        hipError_t e = launch_chunk_table(a.N, a.T, a.cu_seqlens, reinterpret_cast<int32_t *>(ws + w.off_meta),
                                          reinterpret_cast<int32_t *>(ws + w.off_cu),
                                          reinterpret_cast<int32_t *>(ws + w.off_row0),
                                          reinterpret_cast<int32_t *>(ws + w.off_rowtok),
                                          reinterpret_cast<int32_t *>(ws + w.off_rowlen), w.seg_chunks,
                                          reinterpret_cast<int32_t *>(ws + w.off_segfirst),
                                          reinterpret_cast<int32_t *>(ws + w.off_segcnt),
                                          reinterpret_cast<int32_t *>(ws + w.off_segtab), st, !short_call);
        if (e != hipSuccess) return e;
    }
    // Few tokens per sequence (e.g. appending to resident states): one kernel
    // reads and writes each state once and no chunk intermediates are formed
    // (G6, or the token-serial G5).
    if (short_call) {   // (the table pass above only checked cu_seqlens)
        int32_t *meta = reinterpret_cast<int32_t *>(ws + w.off_meta);
        return use_chunk_small(a) ? launch_chunk_small(a, meta, st) : launch_chunk_short(a, meta, st);
    }
    switch (a.in_dtype) {
    case DT_FP32: return launch_typed<float, float>(a, w, st);
    case DT_BF16: return launch_typed<bf16_t, _Float16>(a, w, st);
    case DT_FP16: return launch_typed<_Float16, _Float16>(a, w, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
