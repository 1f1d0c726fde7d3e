// kda_prep.hip -- token-parallel half of the chunked forward pass (gfx950).
//
// One workgroup per (chunk, head), one wave per 16-token block of the chunk.
// It fuses the gate activation, the sigmoid of beta, the in-chunk cumulative
// decay, the q/k L2 norms, the intra-chunk matrices (bf16 MFMA over K), the
// exact inverse (I + A)^-1 by the doubling product, and writes the chunk
// record that kda_recur consumes (layout in kda_common.h).
//
// The split into a token-parallel kernel and a head-parallel recurrence
// follows the FlashKDA summary (discuss.pytorch.kr, section "커널 퓨전(Kernel
// Fusion) 전략의 분리"): gate activation, L2 norm, decay and the matrix inverse
// go in the first kernel; the chunked delta recurrence and the output
// projection in the second.  The gate, beta and norm definitions follow the
// parameter table of the same page (section "FlashKDA의 KDA 연산 구조"); the
// chunk size and the exact 16x16 inverse follow its section "Flash Linear
// Attention과 비교".
#include <hip/hip_ext.h>

#include "kda_common.h"
#include "kda_launch.h"
#include "kda_ops.h"

namespace kda {

// One workgroup per (chunk, head) with one wave per 16-token block.  Lane
// l = m + 16 g of wave b owns token row 16 b + m of the chunk and, for every
// k-step j, the 8 contiguous channels 32 j + 8 g .. +7: exactly the row-m
// slice of a 16x16x32 MFMA fragment.  Every intra-block product therefore
// reads its operands straight from registers, and the q/k/g loads and the
// nKG/QG record stores are 16-byte vectors.
//
//  - gate:   log2 a = max(lb, -exp(A_log[h]) softplus(g + dt_bias)) log2(e)
//  - cumsum: inclusive prefix over a block's 16 rows = 16-lane DPP row scan;
//            block totals are exchanged through LDS
//  - norms:  sum of squares over the 4 lane groups of a row (2 xor shuffles)
//  - in-block A, A^T, Aqk^T: bf16 MFMA over K with the factored decays
//            (k^ Gam)(k^/Gam)^T, exact in range because |G| <= 80 in a block
//            (GDN: products of k^, q^ times exp(G_r - G_j) <= 1 per element)
//  - cross-block A10, Aqk10^T (two blocks): (k^ Gam_loc1)(k^ Gam_end0/Gam0)^T,
//            both factors <= 1
//  - (I + A)^-1 per block by fp32 forward substitution (T (I + A) = I, one
//    row of T per lane, A broadcast from LDS).  A power series of A (the
//    Neumann / doubling form on the FlashKDA page) is exact in exact
//    arithmetic because A^16 = 0, but with near-parallel keys and beta ~ 1
//    its partial sums reach ~10^3 before cancelling to O(1), so low-precision
//    operands lose the result; substitution only ever forms entries of T.
//    Two blocks: T10 = -T11 A10 T00 on fp32 MFMA, with the primitive
//    M(P, Q) = P^T Q on D-layout operands (the D layout of P read as an A
//    operand is P^T), so no product needs a layout change.

// BREC: also write the reverse-pass record (BRec, kda_common.h) for the
// backward pass: the same matrices, transposed through LDS.
template <int K, bool GDN, bool BREC>
__global__ __launch_bounds__(64 * NB) void kda_prep_kernel(PrepArgs a) {
    static_assert(!BREC || NB == 2, "the reverse-pass record is written for 32-token chunks");
    constexpr int KS = K / 32;  // 16-byte channel slices per lane
    using R = Rec<K>;
    __shared__ __attribute__((aligned(16))) uint16_t kdt_s[C * K];   // KdT transpose
    __shared__ __attribute__((aligned(16))) float gend_s[NB][K];     // block log2-decay totals
    __shared__ __attribute__((aligned(16))) bf16x8 kd0_s[NB == 2 ? KS * 64 : 1];  // block 0
    __shared__ __attribute__((aligned(16))) float t00_s[256];        // block 0's T, row-major
    __shared__ __attribute__((aligned(16))) float a_s[NB][256];      // each block's A, row-major
    __shared__ float beta0_s[16];
    __shared__ float dmax_s[NB];  // per block: sum over rows of the row's largest log2 decay
    __shared__ __attribute__((aligned(16))) float eg_s[NB][K];  // KDA: 2^(block total) per channel
    // KDA, per block and channel: the factor its KG and QG carry from the
    // blocks before it and the one its Kd carries from the blocks after it
    __shared__ __attribute__((aligned(16))) float ebef_s[NB][K];
    __shared__ __attribute__((aligned(16))) float eaft_s[NB][K];
    // reverse-pass record only: QG^T, nKG^T (layout of KdT), Aqk and Tb rows
    __shared__ __attribute__((aligned(16))) uint16_t qgt_s[BREC ? C * K : 1];
    __shared__ __attribute__((aligned(16))) uint16_t nkgt_s[BREC ? C * K : 1];
    __shared__ __attribute__((aligned(16))) uint16_t aqk_s[BREC ? C * C : 1];  // [r][s]
    __shared__ __attribute__((aligned(16))) uint16_t tb_s[BREC ? C * C : 1];   // [r][s]

    // heads fastest: the workgroups in flight together read whole token rows
    // ([H, K] contiguous) rather than one head's 256 bytes of many rows
    const int slot = blockIdx.x / a.H;
    const int h = blockIdx.x % a.H;
    const int blk = threadIdx.x >> 6;  // this wave's 16-token block
    const int L = threadIdx.x & 63, m = L & 15, g = L >> 4;

    // ---- locate the chunk: sequence n with chunk_off[n] <= slot < chunk_off[n+1]
    int n;
    if (!a.packed) {
        n = slot / ((a.T + C - 1) / C);  // launched only when T > 0
        if (n >= a.n_seqs) return;       // uniform over the workgroup
    } else {
        if (slot >= a.chunk_off[a.n_seqs]) return;
        int lo = 0, hi = a.n_seqs;  // invariant: chunk_off[lo] <= slot < chunk_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.chunk_off[mid] <= slot) lo = mid; else hi = mid;
        }
        n = lo;
    }
    int64_t t0, t1;
    int s0, s1;
    seq_span(a, n, t0, t1, s0, s1);
    const int64_t start = t0 + (int64_t)C * (slot - s0);  // first token of the chunk
    const int nvalid = (int)min((int64_t)C, t1 - start);   // >= 1
    const int row_in_chunk = 16 * blk + m;
    const bool valid = row_in_chunk < nvalid;

    // ---- every global load up front, from an always-valid row (padding rows
    // re-read the chunk's first row and are zeroed by value), so the wave
    // waits for memory once; q, k, g stay packed bf16 until their slice is used
    const int64_t lrow = (start + (valid ? row_in_chunk : 0)) * a.H + h;
    u32x4 qr[KS], kr[KS], gr[KS];
    floatx4 dtr[KS][2];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int c = 32 * j + 8 * g;
        qr[j] = *reinterpret_cast<const u32x4*>(a.q + lrow * K + c);
        kr[j] = *reinterpret_cast<const u32x4*>(a.k + lrow * K + c);
        if constexpr (!GDN) {
            gr[j] = *reinterpret_cast<const u32x4*>(a.g_kda + lrow * K + c);
            dtr[j][0] = *reinterpret_cast<const floatx4*>(a.dt_bias + (int64_t)h * K + c);
            dtr[j][1] = *reinterpret_cast<const floatx4*>(a.dt_bias + (int64_t)h * K + c + 4);
        }
    }
    const float braw = bf2f(a.beta[lrow]);
    const float graw = GDN ? a.g_gdn[lrow] : 0.f;
    const float rate = GDN ? 0.f : exp2_hw(a.A_log[h] * LOG2E);
    // beta: KDA logits through the sigmoid, GDN probabilities as given; 0 on padding
    const float b = valid ? (GDN ? braw : sigmoid_f(braw)) : 0.f;
    const float vmask = valid ? 1.f : 0.f;

    // ---- L2 norms: a row's channels live in lanes m, m+16, m+32, m+48.
    // Padding rows get zero scales, which zeroes every q^ and k^ product
    // below (their q and k are a real row's, so finite).
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        float x[8], y[8];
        unpack8(qr[j], x);
        unpack8(kr[j], y);
#pragma unroll
        for (int e = 0; e < 8; ++e) { sq += x[e] * x[e]; sk += y[e] * y[e]; }
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    sk += __shfl_xor(sk, 16, 64);
    sk += __shfl_xor(sk, 32, 64);
    const float iq = rsq_hw(sq + NORM_EPS) * vmask, ik = rsq_hw(sk + NORM_EPS) * vmask;

    // ---- in-block inclusive prefix sums of the log2 decay (padding rows add 0)
    float G[KS][8];  // KDA: per channel; GDN uses G[0][0] as the row's value
    // Also the chunk's bound on its state transition: for one token,
    // ||(I - b k^ k^T) Diag(a)||_2 <= max_c a_c (k^ is a unit vector and b is in
    // [0, 1]), so the sum over the chunk's tokens of max_c log2 a_c bounds the
    // log2 norm of the chunk's transition.  Sequence splitting uses it to skip
    // propagating a state through a segment that provably forgets it.
    float rowmax;
    if constexpr (GDN) {
        rowmax = valid ? graw * LOG2E : 0.f;
        G[0][0] = row_scan16(rowmax);
        if (m == 15 && g == 0) gend_s[blk][0] = G[0][0];
    } else {
        // log2 a = max(lb, -rate softplus(y)) log2(e) with softplus(y) = max(y, 0)
        // + ln2 log2(1 + 2^(-|y| log2 e)), so (ln2 log2 e = 1)
        //   log2 a = max(lb log2 e, -rate log2(e) max(y, 0) - rate log2(1 + t)).
        // On padding rows the three per-row constants are zero, which makes
        // log2 a = 0 with no per-element mask (y is finite there: the row is a
        // real row re-read).
        const float lb2 = a.lower_bound * LOG2E * vmask;
        const float c1 = -rate * LOG2E * vmask, c2 = -rate * vmask;
        rowmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            float x[8];
            unpack8(gr[j], x);
            const floatx4 d0 = dtr[j][0], d1 = dtr[j][1];
            const float dv[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y = x[e] + dv[e];
                const float t = exp2_hw(-fabsf(y) * LOG2E);
                const float la = fmaxf(lb2, fmaf(c1, fmaxf(y, 0.f), c2 * log2_hw(1.f + t)));
                rowmax = fmaxf(rowmax, la);
                G[j][e] = la;
            }
        }
        row_scan16_n<KS * 8>(&G[0][0]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            if (m == 15) {  // the block total of these channels
                const floatx4 lo = {G[j][0], G[j][1], G[j][2], G[j][3]};
                const floatx4 hi = {G[j][4], G[j][5], G[j][6], G[j][7]};
                *reinterpret_cast<floatx4*>(&gend_s[blk][32 * j + 8 * g]) = lo;
                *reinterpret_cast<floatx4*>(&gend_s[blk][32 * j + 8 * g + 4]) = hi;
            }
        }
        rowmax = fmaxf(rowmax, __shfl_xor(rowmax, 16, 64));
        rowmax = fmaxf(rowmax, __shfl_xor(rowmax, 32, 64));
    }
    {
        const float dsum = row_scan16(rowmax);  // rows 0..m of the block
        if (m == 15 && g == 0) dmax_s[blk] = dsum;
    }
    __syncthreads();
    if constexpr (!GDN) {
        // 2^(block total) per channel, once per workgroup rather than per row
        for (int c = threadIdx.x; c < NB * K; c += 64 * NB) eg_s[c / K][c % K] = exp2_hw(gend_s[c / K][c % K]);
        for (int c = threadIdx.x; c < K; c += 64 * NB) {
            ebef_s[0][c] = 1.f;
            eaft_s[NB - 1][c] = 1.f;
            if constexpr (NB == 2) {
                ebef_s[1][c] = exp2_hw(gend_s[0][c]);
                eaft_s[0][c] = exp2_hw(gend_s[1][c]);
            }
        }
    }
    if (threadIdx.x == 0) {
        float d = 0.f;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) d += dmax_s[bb];
        a.bound[(int64_t)slot * a.H + h] = d;
    }
    if constexpr (!GDN) __syncthreads();

    // ---- decay factors, record fragments, in-block (and cross-block) products.
    // mfma32(X, Y) gives D = X Y^T: lane (n, g) holds element i of D at row
    // 4g + i, column n.
    unsigned char* rec = a.rec + ((int64_t)slot * a.H + h) * R::BYTES;
    floatx4 dA = {0.f, 0.f, 0.f, 0.f}, dQT = dA, dX = dA, dXQT = dA;
    bf16x8 kgl_f[KS], qgl_f[KS];  // block 1's local KG and QG (cross-block products)
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        float qn[8], kn[8];
        unpack8(qr[j], qn);
        unpack8(kr[j], kn);
#pragma unroll
        for (int e = 0; e < 8; ++e) { qn[e] *= iq; kn[e] *= ik; }
        float kg[8], qg[8], kgl[8], qgl[8], kil[8], kdl[8], kd[8];
        if constexpr (GDN) {
            // any log decay <= 0: only exponents <= 0 are formed
            float gown[8], goth[8];  // this block's and the other block's totals
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gown[e] = gend_s[blk][0];
                goth[e] = NB == 2 ? gend_s[1 - blk][0] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float Gl = G[0][0];
                const float gl = exp2_hw(Gl);
                kgl[e] = kn[e] * gl;
                qgl[e] = qn[e] * gl;
                kil[e] = kn[e];
                kdl[e] = kn[e] * exp2_hw(gown[e] - Gl);
                const float before = (NB == 2 && blk == 1) ? exp2_hw(goth[e]) : 1.f;
                const float after = (NB == 2 && blk == 0) ? exp2_hw(goth[e]) : 1.f;
                kg[e] = kgl[e] * before;
                qg[e] = qgl[e] * before;
                kd[e] = kdl[e] * after;
            }
        } else {
            // the floor bounds every block's |G| by 80 nats, so 2^-G and the
            // per-channel 2^(total) are finite: Kd = (k^ 2^-G) 2^(own total)
            float eown[8], ebef[8], eaft[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 32 * j + 8 * g + e;
                eown[e] = eg_s[blk][c];
                ebef[e] = ebef_s[blk][c];
                eaft[e] = eaft_s[blk][c];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float Gl = G[j][e];
                const float gl = exp2_hw(Gl);
                kgl[e] = kn[e] * gl;                       // block-local Gam
                qgl[e] = qn[e] * gl;
                kil[e] = kn[e] * exp2_hw(-Gl);
                kdl[e] = kil[e] * eown[e];                 // decay to the block's end
                // global factors: block 1 carries block 0's total decay, block
                // 0's Kd carries block 1's
                kg[e] = kgl[e] * ebef[e];
                qg[e] = qgl[e] * ebef[e];
                kd[e] = kdl[e] * eaft[e];
            }
        }
        {  // -KG: the sign bits of the packed bf16 flipped (exact)
            u32x4 w = __builtin_bit_cast(u32x4, pack8(kg));
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] ^= 0x80008000u;
            *reinterpret_cast<u32x4*>(rec + R::NKG + ((blk * KS + j) * 64 + L) * 16) = w;
        }
        *reinterpret_cast<bf16x8*>(rec + R::QG + ((blk * KS + j) * 64 + L) * 16) = pack8(qg);
        // KdT[t][g'][m'][e'] = Kd[tok(g', e')][rho(t, m')]: transposed through LDS
        // (16-byte units swizzled by st_unit, which the copy-out undoes)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = 2 * j + (e >> 2), mm = 4 * g + (e & 3);
            const int ee = 4 * blk + (m & 3);
            const int tr = ((t * 4 + (m >> 2)) * 16 + mm) * EL + ee;  // record order
            const int ti = st_unit(tr / 8) * 8 + tr % 8;
            kdt_s[ti] = __builtin_bit_cast(uint16_t, (bf16)kd[e]);
            if constexpr (BREC) {
                qgt_s[ti] = __builtin_bit_cast(uint16_t, (bf16)qg[e]);
                nkgt_s[ti] = __builtin_bit_cast(uint16_t, (bf16)(-kg[e]));
            }
        }
        if constexpr (BREC)  // Kd rows, in the layout of nKG
            *reinterpret_cast<bf16x8*>(a.brec + ((int64_t)slot * a.H + h) * BRec<K>::BYTES +
                                       BRec<K>::KD + ((blk * KS + j) * 64 + L) * 16) = pack8(kd);
        const bf16x8 kglf = pack8(kgl), qglf = pack8(qgl);
        if constexpr (GDN) {
            // in-block products of k^ and q^; the decay is applied per element
            const bf16x8 kf = pack8(kn), qf = pack8(qn);
            dA = mfma32(kf, kf, dA);
            dQT = mfma32(kf, qf, dQT);
        } else {
            const bf16x8 kif = pack8(kil);
            dA = mfma32(kglf, kif, dA);    // KG KiG^T
            dQT = mfma32(kif, qglf, dQT);  // KiG QG^T = Aqk^T
        }
        if constexpr (NB == 2) {
            if (blk == 0) kd0_s[j * 64 + L] = pack8(kdl);
            kgl_f[j] = kglf;
            qgl_f[j] = qglf;
        }
    }
    // Gam_C, tile order: channel 32 j + 8 g + e is tile 2j + e/4, row 4g + e%4
    if (blk == 0 && m == 15) {
        float* gp = reinterpret_cast<float*>(rec + R::GAMC);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            float gcv[8];  // the chunk's total decay of this lane's channels
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (GDN) {
                    gcv[e] = exp2_hw(gend_s[0][0] + (NB == 2 ? gend_s[NB - 1][0] : 0.f));
                } else {
                    const int c = 32 * j + 8 * g + e;
                    gcv[e] = eg_s[0][c] * (NB == 2 ? eg_s[NB - 1][c] : 1.f);
                }
            }
            const floatx4 lo = {gcv[0], gcv[1], gcv[2], gcv[3]};
            const floatx4 hi = {gcv[4], gcv[5], gcv[6], gcv[7]};
            *reinterpret_cast<floatx4*>(gp + 32 * j + 4 * g) = lo;
            *reinterpret_cast<floatx4*>(gp + 32 * j + 16 + 4 * g) = hi;
            if constexpr (BREC) {
                float* bp = reinterpret_cast<float*>(a.brec + ((int64_t)slot * a.H + h) * BRec<K>::BYTES +
                                                     BRec<K>::GAMC);
                *reinterpret_cast<floatx4*>(bp + 32 * j + 4 * g) = lo;
                *reinterpret_cast<floatx4*>(bp + 32 * j + 16 + 4 * g) = hi;
            }
        }
    }
    if (blk == 0 && g == 0) beta0_s[m] = b;
    __syncthreads();

    // KdT out, 16 bytes per lane per step
#pragma unroll
    for (int p = 0; p < C * K * 2 / (64 * NB * 16); ++p) {
        const int u = p * 64 * NB + threadIdx.x;  // 16-byte unit of the record
        const int off = u * 16, lo = st_unit(u) * 16;
        *reinterpret_cast<u32x4*>(rec + R::KDT + off) =
            *reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned char*>(kdt_s) + lo);
        if constexpr (BREC) {
            unsigned char* br = a.brec + ((int64_t)slot * a.H + h) * BRec<K>::BYTES;
            *reinterpret_cast<u32x4*>(br + BRec<K>::QGT + off) =
                *reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned char*>(qgt_s) + lo);
            *reinterpret_cast<u32x4*>(br + BRec<K>::NKGT + off) =
                *reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned char*>(nkgt_s) + lo);
        }
    }
    if constexpr (NB == 2) {
        if (blk == 1) {
            // A10 = diag(b1) KG1loc Kd0loc^T and Aqk10^T = Kd0loc QG1loc^T
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                const bf16x8 kd0 = kd0_s[j * 64 + L];  // row m of block 0, as operand
                dX = mfma32(kgl_f[j], kd0, dX);
                dXQT = mfma32(kd0, qgl_f[j], dXQT);
            }
        }
    }

    // ---- masks: the in-block A (row-major into LDS) and Aqk
    float br[4], Gr[4];  // beta and (GDN) prefix log decay of rows 4g .. 4g+3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        br[i] = lane_val(b, 4 * g + i);
        if constexpr (GDN) Gr[i] = lane_val(G[0][0], 4 * g + i);
    }
    floatx4 aq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;  // this element's row; its column is m
        float dec_rm = 1.f, dec_mr = 1.f;
        if constexpr (GDN) {
            dec_rm = r > m ? exp2_hw(Gr[i] - G[0][0]) : 0.f;   // exp(G_r - G_m), r > m
            dec_mr = m >= r ? exp2_hw(G[0][0] - Gr[i]) : 0.f;  // exp(G_m - G_r), m >= r
        }
        a_s[blk][16 * r + m] = m < r ? br[i] * dA[i] * dec_rm : 0.f;  // A[r][m], m < r
        aq[i] = r <= m ? dQT[i] * dec_mr : 0.f;                     // Aqk[m][r], r <= m
    }
    __syncthreads();  // A is in LDS (each wave reads back its own block's)

    // ---- T^T in D layout: lane (m, g) holds T[m][4g + i]
    const floatx4 TT = tri_inv_row(a_s[blk], m, g);
    if constexpr (NB == 2) {
        if (blk == 0)  // block 0's T row-major, for the coupling block
            *reinterpret_cast<floatx4*>(&t00_s[16 * m + 4 * g]) = TT;
    }

    // ---- records Aqk (output block blk) and Tb (row block blk)
    floatx4 aq_lo = aq, aq_hi = {0.f, 0.f, 0.f, 0.f};
    floatx4 tb_lo, tb_hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) tb_lo[i] = br[i] * TT[i];  // Tb[m][4g+i] = T[m][4g+i] b_{4g+i}
    if constexpr (NB == 2) {
        __syncthreads();  // T00 and the block-0 betas are in LDS
        if (blk == 1) {
            // T10^T = -T00^T A10^T T11^T = -M(T00, M(A10, T11^T))
            floatx4 A10;
#pragma unroll
            for (int i = 0; i < 4; ++i) A10[i] = br[i] * dX[i];  // A10[r][j] = b1_r (...)
            floatx4 T00;  // D layout: T00[4g + i][m]
#pragma unroll
            for (int i = 0; i < 4; ++i) T00[i] = t00_s[16 * (4 * g + i) + m];
            const floatx4 Z = mt(A10, TT);
            const floatx4 T10T = mt(T00, Z);
            // row block 1: columns of block 0 then block 1
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tb_hi[i] = tb_lo[i];                              // Tb11
                tb_lo[i] = -beta0_s[4 * g + i] * T10T[i];         // Tb10
                aq_hi[i] = aq[i];                                 // Aqk11
                aq_lo[i] = dXQT[i];                               // Aqk10 (all j < r)
            }
        }
    }
    *reinterpret_cast<bf16xEL*>(rec + R::AQK + (blk * 64 + L) * (2 * EL)) = pack_tok(aq_lo, aq_hi);
    *reinterpret_cast<bf16xEL*>(rec + R::TB + (blk * 64 + L) * (2 * EL)) = pack_tok(tb_lo, tb_hi);
    if constexpr (BREC) {
        // rows 16 blk + m of Aqk and Tb through LDS, then their columns:
        // AQKT[a][g][n][e] = Aqk[tok(g,e)][16a+n], TBT likewise
        const u32x4 wa = __builtin_bit_cast(u32x4, pack_tok(aq_lo, aq_hi));
        const u32x4 wt = __builtin_bit_cast(u32x4, pack_tok(tb_lo, tb_hi));
#pragma unroll
        for (int e = 0; e < EL; ++e) {
            const int s = 16 * (e >> 2) + 4 * g + (e & 3);
            aqk_s[(16 * blk + m) * C + s] = (uint16_t)(wa[e >> 1] >> (16 * (e & 1)));
            tb_s[(16 * blk + m) * C + s] = (uint16_t)(wt[e >> 1] >> (16 * (e & 1)));
        }
        __syncthreads();
        u32x4 oa, ot;
#pragma unroll
        for (int u = 0; u < EL / 2; ++u) {
            const int e0 = 2 * u, e1 = 2 * u + 1;
            const int r0 = 16 * (e0 >> 2) + 4 * g + (e0 & 3), r1 = 16 * (e1 >> 2) + 4 * g + (e1 & 3);
            oa[u] = (uint32_t)aqk_s[r0 * C + 16 * blk + m] | ((uint32_t)aqk_s[r1 * C + 16 * blk + m] << 16);
            ot[u] = (uint32_t)tb_s[r0 * C + 16 * blk + m] | ((uint32_t)tb_s[r1 * C + 16 * blk + m] << 16);
        }
        unsigned char* br = a.brec + ((int64_t)slot * a.H + h) * BRec<K>::BYTES;
        *reinterpret_cast<u32x4*>(br + BRec<K>::AQKT + (blk * 64 + L) * (2 * EL)) = oa;
        *reinterpret_cast<u32x4*>(br + BRec<K>::TBT + (blk * 64 + L) * (2 * EL)) = ot;
    }
}

// Sequence table: seq_start[0..N] (flattened token offsets) and
// chunk_off[0..N] (prefix sums of ceil(len / C)).  The sequence ends are
// clamped into [0, total_tokens] and made non-decreasing by a running
// maximum, so a malformed cu_seqlens can never send a later access out of
// bounds: lengths stay >= 0, they sum to at most total_tokens, and the chunk
// count stays within ceil(total_tokens / C) + N.
__device__ __forceinline__ int32_t block_scan(int32_t v, int32_t* buf, bool use_max) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int32_t o = tid >= d ? buf[tid - d] : (use_max ? INT32_MIN : 0);
        __syncthreads();
        buf[tid] = use_max ? max(buf[tid], o) : buf[tid] + o;
        __syncthreads();
    }
    return buf[tid];
}

__global__ __launch_bounds__(256) void kda_seq_table_kernel(const int32_t* cu, int32_t n_seqs,
                                                            int32_t T, int64_t total_tokens,
                                                            int32_t* seq_start,
                                                            int32_t* chunk_off) {
    __shared__ int32_t buf[256];
    __shared__ int32_t ends[256];
    const int tid = threadIdx.x;
    int32_t prev_end = 0, carry = 0;  // identical in every thread
    if (tid == 0) {
        seq_start[0] = 0;
        chunk_off[0] = 0;
    }
    for (int base = 0; base < n_seqs; base += 256) {
        const int i = base + tid;  // sequence i spans [end_{i-1}, end_i)
        int64_t e = prev_end;
        if (i < n_seqs) e = cu ? (int64_t)cu[i + 1] : (int64_t)(i + 1) * T;
        e = min(max(e, (int64_t)prev_end), total_tokens);
        const int32_t end = block_scan((int32_t)e, buf, true);
        ends[tid] = end;
        __syncthreads();
        const int32_t begin = tid == 0 ? prev_end : ends[tid - 1];
        const int32_t chunks = (end - begin + C - 1) / C;
        const int32_t off = block_scan(chunks, buf, false);
        if (i < n_seqs) {
            seq_start[i + 1] = end;
            chunk_off[i + 1] = carry + off;
        }
        carry += buf[255];
        prev_end = ends[255];
        __syncthreads();
    }
}

void launch_seq_table(const int32_t* cu, int32_t n_seqs, int32_t T, int64_t total_tokens,
                      int32_t* seq_start, int32_t* chunk_off, hipStream_t stream) {
    hipLaunchKernelGGL(kda_seq_table_kernel, dim3(1), dim3(256), 0, stream, cu, n_seqs, T,
                       total_tokens, seq_start, chunk_off);
}

template <int K, bool GDN>
void launch_prep_t(const PrepArgs& a, int n_slots, hipStream_t stream, const LaunchEvents* ev) {
    const dim3 grid(n_slots * a.H), block(64 * NB);
    auto go = [&](auto kernel) {
        if (ev) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev->start, ev->stop, 0, a);
        else hipLaunchKernelGGL(kernel, grid, block, 0, stream, a);
    };
    if (a.brec) go(kda_prep_kernel<K, GDN, true>);
    else go(kda_prep_kernel<K, GDN, false>);
}

void launch_prep(const PrepArgs& a, int K, bool gdn, int n_slots, hipStream_t stream,
                 const LaunchEvents* ev) {
    if (K == 128) {
        if (gdn) launch_prep_t<128, true>(a, n_slots, stream, ev);
        else launch_prep_t<128, false>(a, n_slots, stream, ev);
    } else {
        if (gdn) launch_prep_t<64, true>(a, n_slots, stream, ev);
        else launch_prep_t<64, false>(a, n_slots, stream, ev);
    }
}

int record_bytes(int K) { return K == 128 ? Rec<128>::BYTES : Rec<64>::BYTES; }

}  // namespace kda
