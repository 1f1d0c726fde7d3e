// kda_common.h -- shared device definitions for the gfx950 KDA / GDN kernels.
//
// Chunk size, MFMA operand layouts, the per-chunk record written by kda_prep
// and read by kda_recur, and the transcendental helpers built on the gfx950
// hardware instructions (v_exp_f32 = 2^x, v_log_f32 = log2 x, v_rcp_f32,
// v_rsq_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

// Tokens per chunk: C = 16 NB, processed as NB blocks of 16 tokens.
// The FlashKDA summary (discuss.pytorch.kr, section "Flash Linear Attention과
// 비교") motivates the 16-token block: with the gate floored at -5 a 16-token
// cumulative decay stays within 16*5 = 80 < ln(FLT_MAX) ~ 88.7, so the
// factored in-block decays exp(+-G) fit the fp32/bf16 exponent range without
// rescaling, and the 16x16 inverse is cheap.  Larger chunks (FLA's default is
// 64) need the rescaling that page mentions; here it is per 16-token block:
// every cross-block product is formed from two factors that are both <= 1
// (decay from the earlier block's end), and the chunk's (I + A)^-1 is block
// lower triangular.  NB = 2 halves the sequential steps of the recurrence
// and lets its state update run on full-rate 16x16x32 MFMA.
#ifndef KDA_CHUNK_BLOCKS
#define KDA_CHUNK_BLOCKS 2
#endif
constexpr int NB = KDA_CHUNK_BLOCKS;
static_assert(NB == 1 || NB == 2, "chunks of 16 or 32 tokens");
constexpr int C = 16 * NB;
// elements per lane of an operand that contracts over the chunk's tokens:
// token k-slot (g, e) of such an operand is 16 (e / 4) + 4 g + (e % 4)
constexpr int EL = 4 * NB;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NORM_EPS = 1e-6f;

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;  // one 16-byte slice

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16].
// Lane l = r + 16 g (r = l % 16, g = l / 16) holds A row r and B column r,
// eight k-slots each; element e of lane group g of A multiplies element e of
// lane group g of B, so any assignment of real k indices to (g, e) works as
// long as A and B use the same one.  D: lane l holds D[4g + i][r], i = 0..3.
__device__ __forceinline__ floatx4 mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_bf16: lane l = r + 16 g holds A[r][4g + i], B[4g + i][r];
// D as above.  The D layout of a 16x16 result therefore is exactly the B
// layout of the next 16x16x16 product that contracts over D's row index.
__device__ __forceinline__ floatx4 mfma16(bf16x4 a, bf16x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                     __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}

// Operand that contracts over the chunk's tokens: EL bf16 per lane.
typedef __attribute__((ext_vector_type(EL))) __bf16 bf16xEL;
// D += A B over the C tokens: 16x16x16 for one block, 16x16x32 for two.
__device__ __forceinline__ floatx4 mfma_tok(bf16xEL a, bf16xEL b, floatx4 c) {
#if KDA_CHUNK_BLOCKS == 1
    return mfma16(a, b, c);
#else
    return mfma32(a, b, c);
#endif
}

__device__ __forceinline__ bf16x4 to_bf16x4(floatx4 x) {
    bf16x4 r;
    r[0] = (bf16)x[0];
    r[1] = (bf16)x[1];
    r[2] = (bf16)x[2];
    r[3] = (bf16)x[3];
    return r;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).  Array
// indices derived from I are constants from the first optimisation pass on,
// so register arrays indexed by them never fall back to scratch memory.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float rsq_hw(float x) { return __builtin_amdgcn_rsqf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log(1 + e^-|x|), with both
// exponentials taken base 2.
__device__ __forceinline__ float softplus_f(float x) {
    float t = exp2_hw(-fabsf(x) * LOG2E);
    return fmaxf(x, 0.f) + LN2 * log2_hw(1.f + t);
}
// sigmoid(x) = 1 / (1 + e^-x); saturates to exactly 0 or 1 for large |x|.
__device__ __forceinline__ float sigmoid_f(float x) { return rcp_hw(1.f + exp2_hw(-x * LOG2E)); }

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// ---------------------------------------------------------------- record
// Per (chunk slot, head) record written by kda_prep and read by kda_recur.
// All matrices are stored in the exact per-lane order of the MFMA operand
// that consumes them, so kda_recur reads each fragment with one 8- or
// 16-byte access per lane and the whole record is one contiguous stream.
//
// Within a chunk (token r), G[r][c] = sum_{s<=r} log a_s[c] and Gam = exp(G):
//   nKG  = -(k^ * Gam)           [C x K]  per 16-token block: A operand of
//                                         16x16x32 against S
//   QG   =   q^ * Gam            [C x K]  per block: B operand against S^T
//   KdT  = (k^ * Gam_C / Gam)^T  [K x C]  per 16-channel state tile: A operand
//                                         contracting over the C tokens
//   Aqk  = tril(QG (k^/Gam)^T)   [C x C]  per 16-token output block: B operand
//                                         (transposed) contracting over tokens
//   Tb   = (I + A)^-1 diag(b)    [C x C]  per 16-token row block: A operand of
//                                         U' = Tb (V - KG S)
//   GamC = Gam at the chunk's last token, fp32 [K] in tile-channel order
// with A[r][j] = b_r sum_c (k^ Gam)[r][c] (k^/Gam)[j][c] for j < r.
// Token k-slots follow EL above; channel orders follow below.
// Channel orders.  Inside a 16x16x32 fragment that contracts over channels,
// k-step j, lane group g and element e hold channel 32 j + 8 g + e (8
// contiguous channels per lane, so prep loads and stores them as 16-byte
// vectors).  kda_recur keeps the state
// as K/16 tiles of 16 channels in MFMA D layout (lane group g holds tile rows
// 4g..4g+3); tile t, row r holds channel
//   rho(t, r) = 32 (t / 2) + 8 (r / 4) + 4 (t % 2) + (r % 4),
// chosen so that tiles 2j and 2j+1, elements 0..3 of lane group g, are
// exactly channels 32 j + 8 g + 0..7: the fp32 state tiles become the bf16
// B (and A) operand of the next chunk's 16x16x32 products with no data
// movement.  KdT and GamC are stored in tile order.
template <int K>
struct Rec {
    static constexpr int KSTEPS = K / 32;      // 16x16x32 k-steps over channels
    static constexpr int KTILES = K / 16;      // 16-channel state tiles
    static constexpr int NKG = 0;              // bf16 [NB][KSTEPS][4][16][8]
    static constexpr int QG = NKG + C * K * 2; // bf16 [NB][KSTEPS][4][16][8]
    static constexpr int KDT = QG + C * K * 2; // bf16 [KTILES][4][16][EL]:
                                               //   [t][g][m][e] = Kd[tok(g,e)][rho(t,m)]
    static constexpr int AQK = KDT + C * K * 2;  // bf16 [NB][4][16][EL]:
                                                 //   [a][g][n][e] = Aqk[16a+n][tok(g,e)]
    static constexpr int TB = AQK + C * C * 2;   // bf16 [NB][4][16][EL]:
                                                 //   [b][g][m][e] = Tb[16b+m][tok(g,e)]
    static constexpr int GAMC = TB + C * C * 2;  // fp32 [K]: [t][r] = Gam_C[rho(t,r)]
    static constexpr int BYTES = GAMC + K * 4;
};

// Per (chunk slot, head) record of the reverse pass: the same matrices as Rec,
// transposed for the adjoint recurrence (kda_prep writes both).
// With dS' the gradient of the state leaving the chunk and dO its output
// gradient, the reverse step is
//   dU = Kd dS' + scale Aqk^T dO,  dV = Tb^T dU,
//   dS = Diag(Gam_C) dS' + scale QG^T dO + nKG^T dV,
// so Kd is needed row-major (A operand over channels, layout of Rec::NKG) and
// QG, nKG, Aqk, Tb transposed (A operands over tokens).
template <int K>
struct BRec {
    static constexpr int KSTEPS = K / 32;
    static constexpr int KTILES = K / 16;
    static constexpr int KD = 0;                  // bf16 [NB][KSTEPS][4][16][8]
    static constexpr int QGT = KD + C * K * 2;    // bf16 [KTILES][4][16][EL]:
                                                  //   [t][g][m][e] = QG[tok(g,e)][rho(t,m)]
    static constexpr int NKGT = QGT + C * K * 2;  // same layout, nKG
    static constexpr int AQKT = NKGT + C * K * 2; // bf16 [NB][4][16][EL]:
                                                  //   [a][g][n][e] = Aqk[tok(g,e)][16a+n]
    static constexpr int TBT = AQKT + C * C * 2;  // bf16 [NB][4][16][EL]:
                                                  //   [b][g][m][e] = Tb[tok(g,e)][16b+m]
    static constexpr int GAMC = TBT + C * C * 2;  // fp32 [K], as in Rec
    static constexpr int BYTES = GAMC + K * 4;
    static_assert(BYTES == Rec<K>::BYTES, "the stage layout of kda_recur assumes equal sizes");
};

// Position of chunk token s among the EL k-slots of a token operand: the slot
// (g, e) with tok(g, e) = 16 (e / 4) + 4 g + e % 4 = s sits at index 8 g + e
// (two blocks; with one block, 4 g + e).
__host__ __device__ constexpr int tok_pos(int s) {
    return EL * ((s & 15) >> 2) + 4 * (s >> 4) + (s & 3);
}

// channel of element e of lane group g in k-step j of a 16x16x32 fragment
__host__ __device__ constexpr int frag_channel(int j, int g, int e) { return 32 * j + 8 * g + e; }
// channel of row r of state tile t
__host__ __device__ constexpr int tile_channel(int t, int r) {
    return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}

// Flattened token range [t0, t1) and chunk-slot range [s0, s1) of sequence n.
// Fixed-length batches need no table: sequence n is tokens [n T, (n+1) T)
// and slots [n ceil(T/C), (n+1) ceil(T/C)).
template <class Args>
__device__ __forceinline__ void seq_span(const Args& a, int n, int64_t& t0, int64_t& t1, int& s0,
                                         int& s1) {
    if (!a.packed) {
        const int nt = (a.T + C - 1) / C;
        t0 = (int64_t)n * a.T;
        t1 = t0 + a.T;
        s0 = n * nt;
        s1 = s0 + nt;
    } else {
        t0 = a.seq_start[n];
        t1 = a.seq_start[n + 1];
        s0 = a.chunk_off[n];
        s1 = a.chunk_off[n + 1];
    }
}

}  // namespace kda
