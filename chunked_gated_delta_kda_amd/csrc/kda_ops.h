// kda_ops.h -- device helpers shared by the chunk-preparation code of
// kda_prep.hip and the single-launch forward pass of kda_fused.hip: DPP row
// scans over 16 lanes, bf16 packing, the swizzle of the transposed record
// matrices in LDS, fp32 products of D-layout tiles and the triangular inverse.
#pragma once

#include "kda_common.h"

namespace kda {
namespace ops {

constexpr int ROW_SHR1 = 0x111, ROW_SHR2 = 0x112, ROW_SHR4 = 0x114, ROW_SHR8 = 0x118;


// Inclusive prefix sum over the 16 lanes of each row.  A source lane before
// the row start reads 0 (bound_ctrl), so every step is one v_add_f32_dpp.
__device__ __forceinline__ float row_scan16(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, ROW_SHR1, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0.f, x, ROW_SHR2, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0.f, x, ROW_SHR4, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0.f, x, ROW_SHR8, 0xf, 0xf, true);
    return x;
}

// Many independent scans at once, one DPP step across all of them at a time,
// so no step waits on the one before it in the same scan.
template <int N>
__device__ __forceinline__ void row_scan16_n(float* x) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __builtin_amdgcn_update_dpp(0.f, x[i], ROW_SHR1, 0xf, 0xf, true);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __builtin_amdgcn_update_dpp(0.f, x[i], ROW_SHR2, 0xf, 0xf, true);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __builtin_amdgcn_update_dpp(0.f, x[i], ROW_SHR4, 0xf, 0xf, true);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __builtin_amdgcn_update_dpp(0.f, x[i], ROW_SHR8, 0xf, 0xf, true);
}

__device__ __forceinline__ float lane_val(float x, int src) { return __shfl(x, src, 64); }

// LDS position of 16-byte unit u of the transposed record matrices: one write
// instruction of the transpose touches the units of 4 values of bits 4-5 and
// 4 of bits 2-3 of u; XOR-ing bits 4-5 into bits 0-1 puts those 16 units at
// 16 different 16-byte positions within 256 bytes, i.e. different banks.
__device__ __forceinline__ int st_unit(int u) { return u ^ ((u >> 4) & 3); }

// M(P, Q) = P^T Q for 16 x 16 fp32 matrices given in D layout (lane n + 16 g
// holds rows 4 g .. 4 g + 3 of column n): four v_mfma_f32_16x16x4_f32, the
// i-th contracting over the rows 4 g + i that element i of every lane holds
// (that element read as an A operand is P^T[n][4 g + i], as a B operand
// Q[4 g + i][n]).
__device__ __forceinline__ floatx4 mt(floatx4 p, floatx4 q) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(p[i], q[i], acc, 0, 0, 0);
    return acc;
}

// Row m of T = (I + A)^-1 for a strictly lower-triangular 16 x 16 A stored
// row-major in LDS (a[16 k + j] = A[k][j]), in fp32.  From T (I + A) = I:
// T[m][m] = 1, T[m][j] = 0 for j > m, and for j < m
//   T[m][j] = -sum_{k > j} T[m][k] A[k][j].
// The columns are finished from k = 15 down; each finished T[m][k] is added
// into the pending sums of all columns before it, so the dependent chain is
// one fma per column.  Every lane computes its whole row (lanes of one row
// agree); the result is T[m][4 g + i], i = 0..3: the D layout of T^T.
__device__ __forceinline__ floatx4 tri_inv_row(const float* a, int m, int g) {
    float t[16], s[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        t[j] = j == m ? 1.f : 0.f;
        s[j] = 0.f;
    }
#pragma unroll
    for (int k = 15; k >= 1; --k) {
        if (k < 15) t[k] = k < m ? -s[k] : t[k];
        float row[16];
#pragma unroll
        for (int q = 0; q < (k + 3) / 4; ++q) {
            const floatx4 v = *reinterpret_cast<const floatx4*>(a + 16 * k + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) row[4 * q + e] = v[e];
        }
#pragma unroll
        for (int j = 0; j < k; ++j) s[j] = fmaf(t[k], row[j], s[j]);
    }
    t[0] = 0 < m ? -s[0] : t[0];
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = g == 0 ? t[i] : g == 1 ? t[4 + i] : g == 2 ? t[8 + i] : t[12 + i];
    return r;
}

// Row m of T = (I + A)^-1 (as tri_inv_row) into t[0..15], for a matrix whose
// LDS address may differ between lanes (two matrices inverted at once by two
// lane groups).  Each step reads the next row one step ahead of its use.
__device__ __forceinline__ void tri_inv_rows(const float* a, int m, float (&t)[16]) {
    float s[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        t[j] = j == m ? 1.f : 0.f;
        s[j] = 0.f;
    }
    auto read_row = [&](auto kc, float (&row)[16]) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        static_for<0, (k + 3) / 4>([&](auto q) __attribute__((always_inline)) {
            const floatx4 v = *reinterpret_cast<const floatx4*>(a + 16 * k + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) row[4 * q + e] = v[e];
        });
    };
    float ra[16];
    read_row(std::integral_constant<int, 15>{}, ra);
    static_for<0, 15>([&](auto kk) __attribute__((always_inline)) {
        constexpr int k = 15 - kk;
        float na[16];
        if constexpr (k > 1) read_row(std::integral_constant<int, k - 1>{}, na);
        if constexpr (k < 15) t[k] = k < m ? -s[k] : t[k];
#pragma unroll
        for (int j = 0; j < k; ++j) s[j] = fmaf(t[k], ra[j], s[j]);
        if constexpr (k > 1) {
#pragma unroll
            for (int j = 0; j < k - 1; ++j) ra[j] = na[j];
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    t[0] = 0 < m ? -s[0] : t[0];
}

// T^T in D layout (element i = T[m][4 g + i]) for T = (I + A)^-1, A
// strictly lower-triangular 16 x 16, given row-major in LDS at `a` (which
// this overwrites) and in D layout in `ad`.  With D = diag(T0, T1) the
// inverses of the two diagonal 8 x 8 blocks and E the lower-left 8 x 8 block
// of A, T = D - D E D.  T0 and T1 come from fp32 forward substitution, both
// at once (lanes 0-7 rows of T0, lanes 8-15 rows of T1: seven steps, 28 fmas
// per lane); D is transposed through LDS; D E D is two D-layout products on
// fp32 MFMA (eight v_mfma_f32_16x16x4_f32).
__device__ __forceinline__ floatx4 tri_inv_split_t(float* a, floatx4 ad, int m, int g) {
    const int h = m >> 3, mm = m & 7;
    float t[8], s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        t[j] = j == mm ? 1.f : 0.f;
        s[j] = 0.f;
    }
    const float* ab = a + 136 * h;  // row 8h, column 8h of A
    auto read_row = [&](auto kc, float (&row)[8]) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        static_for<0, (k + 3) / 4>([&](auto q) __attribute__((always_inline)) {
            const floatx4 v = *reinterpret_cast<const floatx4*>(ab + 16 * k + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) row[4 * q + e] = v[e];
        });
    };
    float ra[8];
    read_row(std::integral_constant<int, 7>{}, ra);
    static_for<0, 7>([&](auto kk) __attribute__((always_inline)) {
        constexpr int k = 7 - kk;
        float na[8];
        if constexpr (k > 1) read_row(std::integral_constant<int, k - 1>{}, na);
        if constexpr (k < 7) t[k] = k < mm ? -s[k] : t[k];
#pragma unroll
        for (int j = 0; j < k; ++j) s[j] = fmaf(t[k], ra[j], s[j]);
        if constexpr (k > 1) {
#pragma unroll
            for (int j = 0; j < k - 1; ++j) ra[j] = na[j];
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    t[0] = 0 < mm ? -s[0] : t[0];
    // D's rows over A (its reads are done: LDS accesses of a wave run in order)
    if (g == 0) {
        *reinterpret_cast<floatx4*>(a + 8 * m) = floatx4{t[0], t[1], t[2], t[3]};
        *reinterpret_cast<floatx4*>(a + 8 * m + 4) = floatx4{t[4], t[5], t[6], t[7]};
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    floatx4 dd, y, e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        dd[i] = (r >> 3) == h ? a[8 * r + mm] : 0.f;                        // D[r][m]
        y[i] = (g >> 1) == h ? ((g & 1) ? t[4 + i] : t[i]) : 0.f;          // D[m][r]
        e[i] = (r >= 8 && m < 8) ? ad[i] : 0.f;                             // E[r][m]
    }
    const floatx4 x = mt(e, y);   // E^T D^T
    const floatx4 z = mt(dd, x);  // D^T E^T D^T = (D E D)^T
    return y - z;
}

// t[4 g + i], i = 0..3, for a runtime g in 0..3
__device__ __forceinline__ floatx4 pick4(const float (&t)[16], int g) {
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = g & 1 ? t[4 + i] : t[i];
        const float hi = g & 1 ? t[12 + i] : t[8 + i];
        r[i] = g & 2 ? hi : lo;
    }
    return r;
}

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
    const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f[2 * u] = bf2f(w[u] & 0xffff);
        f[2 * u + 1] = bf2f(w[u] >> 16);
    }
}

__device__ __forceinline__ bf16x8 pack8(const float* f, float s = 1.f) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)(s * f[e]);
    return r;
}

// One token-contraction operand from two 4-element halves (block 0, block 1).
__device__ __forceinline__ bf16xEL pack_tok(floatx4 lo, floatx4 hi) {
    bf16xEL r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = (bf16)lo[i];
        if constexpr (NB == 2) r[4 + i] = (bf16)hi[i];
    }
    return r;
}


// The same for two independent matrices at once (a0, a1), their steps
// interleaved so each hides the other's latency.  Each step reads one row of
// each matrix from LDS one step ahead of its use, and a scheduling barrier
// per step keeps the compiler from hoisting every row read to the top (which
// would hold all 240 entries in registers).
__device__ __forceinline__ void tri_inv_row2(const float* a0, const float* a1, int m, int g,
                                             floatx4& r0, floatx4& r1) {
    float t0[16], s0[16], t1[16], s1[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        t0[j] = t1[j] = j == m ? 1.f : 0.f;
        s0[j] = s1[j] = 0.f;
    }
    // row k of a matrix, entries 0 .. k - 1 (whole 16-byte groups)
    auto read_row = [&](const float* a, auto kc, float (&row)[16]) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        static_for<0, (k + 3) / 4>([&](auto q) __attribute__((always_inline)) {
            const floatx4 v = *reinterpret_cast<const floatx4*>(a + 16 * k + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) row[4 * q + e] = v[e];
        });
    };
    float ra[16], rb[16];
    read_row(a0, std::integral_constant<int, 15>{}, ra);
    read_row(a1, std::integral_constant<int, 15>{}, rb);
    static_for<0, 15>([&](auto kk) __attribute__((always_inline)) {
        constexpr int k = 15 - kk;
        float na[16], nb[16];
        if constexpr (k > 1) {
            read_row(a0, std::integral_constant<int, k - 1>{}, na);
            read_row(a1, std::integral_constant<int, k - 1>{}, nb);
        }
        if constexpr (k < 15) {
            t0[k] = k < m ? -s0[k] : t0[k];
            t1[k] = k < m ? -s1[k] : t1[k];
        }
#pragma unroll
        for (int j = 0; j < k; ++j) {
            s0[j] = fmaf(t0[k], ra[j], s0[j]);
            s1[j] = fmaf(t1[k], rb[j], s1[j]);
        }
        if constexpr (k > 1) {
#pragma unroll
            for (int j = 0; j < k - 1; ++j) {
                ra[j] = na[j];
                rb[j] = nb[j];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    t0[0] = 0 < m ? -s0[0] : t0[0];
    t1[0] = 0 < m ? -s1[0] : t1[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r0[i] = g == 0 ? t0[i] : g == 1 ? t0[4 + i] : g == 2 ? t0[8 + i] : t0[12 + i];
        r1[i] = g == 0 ? t1[i] : g == 1 ? t1[4 + i] : g == 2 ? t1[8 + i] : t1[12 + i];
    }
}

}  // namespace ops
using namespace ops;
}  // namespace kda
