// kda_fused.hip -- the whole chunked forward pass in one launch (gfx950).
//
// The two-stage path (kda_prep then kda_recur) writes a 29 KB record per
// (32-token chunk, head) to HBM and reads it back: at B2 T2048 H32 that round
// trip is larger than the method's own inputs and outputs.  Here one
// workgroup owns a (sequence segment, head) with all V value columns, forms
// each chunk's record in LDS and consumes it there, so HBM sees q, k, g, v,
// beta and the states read once and o and the final states written once.
// The split into a token-parallel stage and a sequential recurrence follows
// the FlashKDA summary (discuss.pytorch.kr, section "커널 퓨전(Kernel Fusion) 전략의
// 분리"); on MI355X the two stages become wave roles inside one workgroup
// instead of two kernels.
//
// Wave roles (one workgroup per CU, two waves per SIMD at K = V = 128):
//   prep waves (K/32): wave p owns channels 32p .. 32p+31 of both 16-token
//     blocks of a chunk.  Lane m + 16g holds tokens m and 16 + m and the eight
//     channels 32p + 8g .. +7, i.e. its slice of a 16x16x32 MFMA operand.  Per
//     chunk, over three iterations: load q, k, g (and beta); the partial sums
//     of squares of q and k over its channels (phase N); the gate, the
//     in-block prefix sums, the decayed operands written into the chunk's LDS
//     record, and partial intra-chunk products over its channels (phase A).
//   compute waves (4): wave w owns V/4 value columns of the [K, V] state in
//     fp32 MFMA accumulators for the whole segment and runs the recurrence of
//     kda_recur.hip on the LDS record.  In turn, one of them also finishes a
//     chunk's record (phase B): the sum of the partial products, the masks and
//     beta, the in-block inverses by forward substitution, the coupling block
//     T10 = -T11 A10 T00, and Tb and Aqk.
// One barrier per iteration.  In iteration i the compute waves run chunk i,
// phase B finishes chunk i+1, phase A fills chunk i+2, phase N covers chunk
// i+3 and the loads of chunk i+4 are issued; three records are live in LDS.
//
// Sequence segments.  A (sequence, head) pair is one chain of chunk steps, so
// long sequences are cut into segments of L chunks that run in parallel.  A
// segment that does not start its sequence starts its recurrence from a zero
// state W chunks early (the warm-up) and checks the bound of those chunks'
// transitions: for one token ||(I - b k^ k^T) Diag(a)||_2 <= max(1, |1 - b|)
// max_c a_c (at most max_c a_c for 0 <= b <= 2), so the state entering the
// segment reaches its first token scaled by at most 2^(the sum over the
// warm-up's tokens of log2 of that factor).  Below 2^bound_limit (2^-40, far
// under fp32 rounding of the state) the zero start is exact to that bound;
// otherwise the segment restarts from the sequence start and its initial
// state.  The FlashQLA summary (section "핵심 기능") describes switching on
// intra-card parallelism when the gate's decay allows it; this is that test,
// made per segment.
#include <hip/hip_ext.h>

#include "kda_common.h"
#include "kda_launch.h"
#include "kda_ops.h"

namespace kda {

namespace {

template <int K, int V>
struct FusedLayout {
    using R = Rec<K>;
    static constexpr int NPW = K / 32;  // prep waves
    static constexpr int NCW = 4;       // compute waves
    static constexpr int CT = V / 64;   // 16-column state tiles per compute wave
    static constexpr int NT = 64 * (NPW + NCW);
    static constexpr int NBUF = 3;      // chunk records in LDS
    // byte offsets
    static constexpr int REC = 0;                                   // [NBUF][R::BYTES]
    static constexpr int PART = REC + NBUF * R::BYTES;              // [2][NPW][6][64] floatx4
    static constexpr int PART_SLOT = NPW * 6 * 64 * 16;
    static constexpr int NORM = PART + 2 * PART_SLOT;               // [2][NPW][64] float
    static constexpr int RMAX = NORM + 2 * NPW * 64 * 4;            // [2][NPW][32] float
    static constexpr int BETA = RMAX + 2 * NPW * 32 * 4;            // [2][32] float
    static constexpr int GTOK = BETA + 2 * 32 * 4;                  // [2][32] float
    static constexpr int TOT = GTOK + 2 * 32 * 4;                   // [NPW][64] float
    static constexpr int AMAT = TOT + NPW * 64 * 4;                 // [2][256] float
    static constexpr int T00 = AMAT + 2 * 256 * 4;                  // [256] float
    static constexpr int MISC = T00 + 256 * 4;                      // bound sum
    static constexpr int BYTES = MISC + 16;
    static_assert(BYTES <= 160 * 1024, "LDS of one CU");
};

// A prep wave's raw inputs for one chunk (block b = 0, 1 of the lane's tokens).
struct PIn {
    u32x4 q[2], k[2], g[2];  // eight bf16 channels each (g: KDA only)
    float gd[2];             // GDN: the tokens' log decay
    uint16_t braw[2];        // beta bits of the two blocks' tokens (kept apart and
                             // unconverted: any operation on them at the load would
                             // wait for the loads right there)
};

// A use of every register of a ring slot that phase A skips: the slot is
// reloaded three iterations later, and without a use on this path the
// compiler's wait for that reload's registers covers the newer loads too.
__device__ __forceinline__ void touch(const PIn& d) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(d.q[b][u]), "v"(d.k[b][u]), "v"(d.g[b][u]));
        asm volatile("" ::"v"(d.gd[b]), "v"((uint32_t)d.braw[b]));
    }
}

// Orders this wave's LDS accesses (writes by some lanes, reads by others).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// The lane index as a value the compiler cannot see through: per-lane
// address arithmetic derived from it is recomputed inside each phase instead
// of hoisted out of the iteration loop and held in registers for its whole
// length (which spills).
__device__ __forceinline__ int opaque_lane() {
    int l = (int)(threadIdx.x & 63);
    asm volatile("" : "+v"(l));
    return l;
}

// s_waitcnt immediates that wait until at most eight (none) vector memory
// loads are outstanding (vmcnt 8 / 0; expcnt and lgkmcnt left at their maximum)
constexpr int VMCNT_8 = 0x0F78;
constexpr int VMCNT_0 = 0x0F70;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// lane 15 of each 16-lane row, broadcast to the row (ds_swizzle bit mode:
// and 0x10, or 0x0f within each half of the wave)
__device__ __forceinline__ float row_last(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1f0));
}

}  // namespace

template <int K, int V, bool GDN>
__global__ __launch_bounds__(64 * (K / 32 + 4)) void kda_fused_kernel(FusedArgs a) {
    using L = FusedLayout<K, V>;
    using R = Rec<K>;
    constexpr int NPW = L::NPW, NCW = L::NCW, CT = L::CT;
    constexpr int KS = K / 32, KT = K / 16;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::BYTES];

    // ---------------------------------------------------------------- segment
    const int h = blockIdx.x % a.H;
    const int vseg = blockIdx.x / a.H;
    int n, fslot;
    int64_t tseq0, tseq1;  // the sequence's tokens
    int c0, c1;            // the segment's chunks (within the sequence)
    if (!a.packed) {
        n = vseg / a.segs_per_seq;
        const int s = vseg % a.segs_per_seq;
        if (n >= a.n_seqs) return;
        tseq0 = (int64_t)n * a.T;
        tseq1 = tseq0 + a.T;
        const int nc = (a.T + C - 1) / C;
        c0 = min(s * a.seg_chunks, nc);
        c1 = min(c0 + a.seg_chunks, nc);
        fslot = s == a.segs_per_seq - 1 ? n : -1;
    } else {
        const int nseg = min(a.vfirst[a.n_seqs], a.n_segs);
        if (vseg >= nseg) return;
        int lo = 0, hi = a.n_seqs;  // vfirst[lo] <= vseg < vfirst[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.vfirst[mid] <= vseg) lo = mid; else hi = mid;
        }
        n = lo;
        // every value read from the tables is kept inside the batch
        tseq0 = min(max((int64_t)a.seq_start[n], (int64_t)0), a.tok_limit);
        tseq1 = min(max((int64_t)a.seq_start[n + 1], tseq0), a.tok_limit);
        const int64_t ts = min(max((int64_t)a.vseq_start[vseg], tseq0), tseq1);
        const int64_t te = min(max((int64_t)a.vseq_start[vseg + 1], ts), tseq1);
        c0 = (int)((ts - tseq0) / C);
        c1 = (int)((te - tseq0 + C - 1) / C);
        fslot = a.final_map[vseg];
        if (fslot >= a.n_seqs) fslot = -1;
    }

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, m = lane & 15, g = lane >> 4;
    const bool is_cw = wave < NCW;
    const int p = wave - NCW;  // prep wave index (>= 0 for prep waves)

    // ---------------------------------------------------- compute-wave state
    const int64_t vstride = (int64_t)a.H * V;
    floatx4 S[CT][KT];
    // column of tile ct, lane lr: with two tiles per wave, tile ct holds the
    // columns of parity ct, so a lane's pair (2 lr, 2 lr + 1) is contiguous
    const int wcol = wave * 16 * CT;
    auto col_of = [&](int ct, int lr) __attribute__((always_inline)) {
        return CT == 2 ? wcol + 2 * lr + ct : wcol + lr;
    };
    // (global accesses: a wave-uniform base pointer and 32-bit lane offsets)
    auto load_state = [&](bool exact) __attribute__((always_inline)) {
        const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4;
        if (exact && a.initial_state) {  // uniform: every load issued before the first wait
            const float* sp = a.initial_state + ((int64_t)n * a.H + h) * K * V;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[ct][t][i] = sp[tile_channel(t, 4 * lg + i) * V + col_of(ct, lr)];
        } else {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[ct][t][i] = 0.f;
        }
    };

    // ------------------------------------------------------- per-head values
    float rate = 0.f, dt[8];
    if constexpr (!GDN) {
        rate = exp2_hw(a.A_log[h] * LOG2E);
        if (!is_cw) {
            const float* dp = a.dt_bias + (int64_t)h * K + 32 * p + 8 * g;
#pragma unroll
            for (int e = 0; e < 8; ++e) dt[e] = dp[e];
        }
    }

    float* const misc = reinterpret_cast<float*>(lds + L::MISC);
    const int W = a.warm_chunks;

    // An attempt computes chunks x0 .. c1 - 1 of the sequence, with outputs
    // from c0 on; attempt 0 starts W chunks early from a zero state (exact
    // when that is the sequence start), attempt 1 (after a failed bound)
    // from the sequence start and its initial state.
    int x0 = 0, n_it = 0, out_from = 0;
    bool exact = true;
    auto begin_attempt = [&](int attempt) __attribute__((always_inline)) {
        x0 = attempt == 0 ? max(0, c0 - W) : 0;  // first chunk computed
        exact = x0 == 0;
        n_it = c1 - x0;                          // chunks computed
        out_from = c0 - x0;                      // first chunk (relative) with outputs
    };
    // the warm-up chunks' bound is complete at iteration out_from (phase B of
    // the last one ran an iteration earlier); every wave reads the same value
    auto failed_bound = [&](int it) __attribute__((always_inline)) {
        return !exact && it == out_from && !(misc[0] < a.bound_limit);
    };

        // ---------------------------------------------------------- prep waves
        // chunk x (relative to x0): its first token
        auto chunk_t0 = [&](int x) __attribute__((always_inline)) { return tseq0 + (int64_t)C * (x0 + x); };
        auto load_in = [&](PIn& d, int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4, lr = m, lg = g;
            (void)lr; (void)lg;
            const int64_t ct0 = chunk_t0(x);
            const int64_t r0 = ct0 * a.H + h;  // the chunk's first (token, head) row
            const uint16_t* qb = a.q + r0 * K;
            const uint16_t* kb = a.k + r0 * K;
            const uint16_t* gb = GDN ? nullptr : a.g_kda + r0 * K;
            const float* gdb = GDN ? a.g_gdn + r0 : nullptr;
            const uint16_t* bt = a.beta + r0;
            const int nvalid = (int)min((int64_t)C, tseq1 - ct0);
            const int cb = 32 * p + 8 * g;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                // padding rows re-read the chunk's first row
                const int r = 16 * b + m < nvalid ? (16 * b + m) * a.H : 0;
                d.q[b] = *reinterpret_cast<const u32x4*>(qb + r * K + cb);
                d.k[b] = *reinterpret_cast<const u32x4*>(kb + r * K + cb);
                if constexpr (!GDN) d.g[b] = *reinterpret_cast<const u32x4*>(gb + r * K + cb);
                else d.gd[b] = gdb[r];
                d.braw[b] = bt[r];
            }
        };
        auto phase_n = [&](const PIn& d, int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4, lr = m, lg = g;
            (void)lr; (void)lg;
            float sq[2], sk[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                sq[b] = 0.f;
                sk[b] = 0.f;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float q0 = bf_lo(d.q[b][u]), q1 = bf_hi(d.q[b][u]);
                    const float k0 = bf_lo(d.k[b][u]), k1 = bf_hi(d.k[b][u]);
                    sq[b] = fmaf(q0, q0, fmaf(q1, q1, sq[b]));
                    sk[b] = fmaf(k0, k0, fmaf(k1, k1, sk[b]));
                }
                sq[b] += __shfl_xor(sq[b], 16, 64);
                sq[b] += __shfl_xor(sq[b], 32, 64);
                sk[b] += __shfl_xor(sk[b], 16, 64);
                sk[b] += __shfl_xor(sk[b], 32, 64);
            }
            if (g == 0) {
                float* nb = reinterpret_cast<float*>(lds + L::NORM) + ((x & 1) * NPW + p) * 64;
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    nb[16 * b + m] = sq[b];
                    nb[32 + 16 * b + m] = sk[b];
                }
            }
        };
        auto phase_a = [&](const PIn& d, int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4, lr = m, lg = g;
            (void)lr; (void)lg;
            const int slot = x & 1;
            unsigned char* rec = lds + L::REC + (x % 3) * R::BYTES;
            const int64_t ct0 = chunk_t0(x);
            const int nvalid = (int)min((int64_t)C, tseq1 - ct0);
            float vmask[2], iq[2], ik[2], bsig[2];
            const float* nb = reinterpret_cast<const float*>(lds + L::NORM) + slot * NPW * 64;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const bool valid = 16 * b + m < nvalid;
                vmask[b] = valid ? 1.f : 0.f;
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int pp = 0; pp < NPW; ++pp) {
                    sq += nb[pp * 64 + 16 * b + m];
                    sk += nb[pp * 64 + 32 + 16 * b + m];
                }
                iq[b] = rsq_hw(sq + NORM_EPS) * vmask[b];
                ik[b] = rsq_hw(sk + NORM_EPS) * vmask[b];
                const float braw = __uint_as_float((uint32_t)d.braw[b] << 16);
                bsig[b] = valid ? (GDN ? braw : sigmoid_f(braw)) : 0.f;
            }
            if (p == 0 && g == 0) {
                float* bs = reinterpret_cast<float*>(lds + L::BETA) + slot * 32;
                bs[m] = bsig[0];
                bs[16 + m] = bsig[1];
            }
            // log2 decays and their in-block prefix sums (padding rows add 0)
            float G[2][8], rmax[2];
            float Gs[2];  // GDN: the token's prefix sum
            if constexpr (GDN) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const float la = vmask[b] > 0.f ? d.gd[b] * LOG2E : 0.f;
                    rmax[b] = la;
                    Gs[b] = row_scan16(la);
                }
                if (p == 0 && g == 0) {
                    float* gt = reinterpret_cast<float*>(lds + L::GTOK) + slot * 32;
                    gt[m] = Gs[0];
                    gt[16 + m] = Gs[1];
                }
            } else {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    // log2 a = max(lb log2 e, -rate log2(e) max(y, 0) - rate log2(1 + 2^(-|y| log2 e)))
                    const float lb2 = a.lower_bound * LOG2E * vmask[b];
                    const float c1v = -rate * LOG2E * vmask[b], c2v = -rate * vmask[b];
                    rmax[b] = -INFINITY;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float x2[2] = {bf_lo(d.g[b][u]), bf_hi(d.g[b][u])};
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int e = 2 * u + hh;
                            const float y = x2[hh] + dt[e];
                            const float t = exp2_hw(-fabsf(y) * LOG2E);
                            const float la = fmaxf(lb2, fmaf(c1v, fmaxf(y, 0.f), c2v * log2_hw(1.f + t)));
                            rmax[b] = fmaxf(rmax[b], la);
                            G[b][e] = la;
                        }
                    }
                }
                row_scan16_n<16>(&G[0][0]);
            }
            // the bound: max over this wave's channels of each token's log2 decay
            if constexpr (!GDN) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    rmax[b] = fmaxf(rmax[b], __shfl_xor(rmax[b], 16, 64));
                    rmax[b] = fmaxf(rmax[b], __shfl_xor(rmax[b], 32, 64));
                }
            }
            if (g == 0) {
                float* rm = reinterpret_cast<float*>(lds + L::RMAX) + (slot * NPW + p) * 32;
                rm[m] = rmax[0];
                rm[16 + m] = rmax[1];
            }
            // per-channel block decays 2^(block total): ef0 (block 0), ef1 (block 1)
            float ef0[8], ef1[8];
            float* tot = reinterpret_cast<float*>(lds + L::TOT) + p * 64;
            if constexpr (GDN) {
                const float t0 = row_last(Gs[0]), t1 = row_last(Gs[1]);
                const float e0 = exp2_hw(t0), e1 = exp2_hw(t1);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ef0[e] = e0;
                    ef1[e] = e1;
                }
            } else {
                if (m == 15) {
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        *reinterpret_cast<floatx4*>(tot + 32 * b + 8 * g) =
                            floatx4{G[b][0], G[b][1], G[b][2], G[b][3]};
                        *reinterpret_cast<floatx4*>(tot + 32 * b + 8 * g + 4) =
                            floatx4{G[b][4], G[b][5], G[b][6], G[b][7]};
                    }
                }
                wave_lds_sync();
                const float e = exp2_hw(tot[lane]);  // one (block, channel) per lane
                wave_lds_sync();
                tot[lane] = e;
                wave_lds_sync();
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const floatx4 v0 = *reinterpret_cast<const floatx4*>(tot + 8 * g + 4 * hh);
                    const floatx4 v1 = *reinterpret_cast<const floatx4*>(tot + 32 + 8 * g + 4 * hh);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ef0[4 * hh + i] = v0[i];
                        ef1[4 * hh + i] = v1[i];
                    }
                }
            }
            // Gamma_C of this wave's channels, tile order (channel 32p + 8g + e is
            // tile 2p + e/4, row 4g + e%4)
            if (m == 15) {
                float* gp = reinterpret_cast<float*>(rec + R::GAMC);
                *reinterpret_cast<floatx4*>(gp + 32 * p + 4 * g) =
                    floatx4{ef0[0] * ef1[0], ef0[1] * ef1[1], ef0[2] * ef1[2], ef0[3] * ef1[3]};
                *reinterpret_cast<floatx4*>(gp + 32 * p + 16 + 4 * g) =
                    floatx4{ef0[4] * ef1[4], ef0[5] * ef1[5], ef0[6] * ef1[6], ef0[7] * ef1[7]};
            }
            // decayed operands, record fragments and the MFMA operands of the
            // partial intra-chunk products:
            //   in-block (ink, inq, ini): KDA (k^ Gam, q^ Gam, k^/Gam) with Gam
            //     from the block start; GDN k^, q^, k^ (its decay is applied per
            //     element in phase B, so no factor 2^-G is ever formed)
            //   coupling (kcp1, qcp1, kd0f): block 1's k^ Gam, q^ Gam and block 0's
            //     k^ Gam_end0 / Gam, both factors <= 1
            bf16x8 ink[2], inq[2], ini[2], kcp1, qcp1, kd0f;
            uint16_t* kdt = reinterpret_cast<uint16_t*>(rec + R::KDT);
            float gtot[2] = {0.f, 0.f};
            if constexpr (GDN) {
                gtot[0] = row_last(Gs[0]);
                gtot[1] = row_last(Gs[1]);
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                float qn[8], kn[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    qn[2 * u] = bf_lo(d.q[b][u]) * iq[b];
                    qn[2 * u + 1] = bf_hi(d.q[b][u]) * iq[b];
                    kn[2 * u] = bf_lo(d.k[b][u]) * ik[b];
                    kn[2 * u + 1] = bf_hi(d.k[b][u]) * ik[b];
                }
                float kg[8], qg[8], kgl[8], qgl[8], kil[8], kdl[8], kd[8];
                float gl_tok = 1.f, gend_tok = 1.f;
                if constexpr (GDN) {
                    gl_tok = exp2_hw(Gs[b]);               // decay from the block start
                    gend_tok = exp2_hw(gtot[b] - Gs[b]);   // decay to the block end
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float gl;
                    if constexpr (GDN) {
                        gl = gl_tok;
                        kil[e] = kn[e];
                        kdl[e] = kn[e] * gend_tok;
                    } else {
                        gl = exp2_hw(G[b][e]);
                        kil[e] = kn[e] * exp2_hw(-G[b][e]);
                        kdl[e] = kil[e] * (b == 0 ? ef0[e] : ef1[e]);
                    }
                    kgl[e] = kn[e] * gl;
                    qgl[e] = qn[e] * gl;
                    if (b == 0) {
                        kg[e] = kgl[e];
                        qg[e] = qgl[e];
                        kd[e] = kdl[e] * ef1[e];
                    } else {
                        kg[e] = kgl[e] * ef0[e];
                        qg[e] = qgl[e] * ef0[e];
                        kd[e] = kdl[e];
                    }
                }
                {  // -KG: the sign bits of the packed bf16 flipped (exact)
                    u32x4 w = __builtin_bit_cast(u32x4, pack8(kg));
#pragma unroll
                    for (int u = 0; u < 4; ++u) w[u] ^= 0x80008000u;
                    *reinterpret_cast<u32x4*>(rec + R::NKG + ((b * KS + p) * 64 + lane) * 16) = w;
                }
                *reinterpret_cast<bf16x8*>(rec + R::QG + ((b * KS + p) * 64 + lane) * 16) = pack8(qg);
                // KdT[t][g'][m'][e'] = Kd[tok(g', e')][rho(t, m')], 16-byte units swizzled
                {
                    const u32x4 w = __builtin_bit_cast(u32x4, pack8(kd));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int t = 2 * p + (e >> 2), mm = 4 * g + (e & 3);
                        const int ee = 4 * b + (m & 3);
                        const int tr = ((t * 4 + (m >> 2)) * 16 + mm) * EL + ee;
                        kdt[st_unit(tr / 8) * 8 + tr % 8] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                    }
                }
                const bf16x8 kglf = pack8(kgl), qglf = pack8(qgl);
                if constexpr (GDN) {
                    ink[b] = pack8(kn);
                    inq[b] = pack8(qn);
                    ini[b] = ink[b];
                } else {
                    ink[b] = kglf;
                    inq[b] = qglf;
                    ini[b] = pack8(kil);
                }
                if (b == 0) kd0f = pack8(kdl);
                if (b == 1) {
                    kcp1 = kglf;
                    qcp1 = qglf;
                }
            }
            // partial products over this wave's 32 channels (D = X Y^T):
            //   0: A00 (in-block K Ki^T)  1: A11  2: Aqk00^T (Ki Q^T)  3: Aqk11^T
            //   4: A10 (KG1 Kd0^T)        5: Aqk10^T (Kd0 QG1^T)
            const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
            floatx4 P[6];
            P[0] = mfma32(ink[0], ini[0], zero);
            P[1] = mfma32(ink[1], ini[1], zero);
            P[2] = mfma32(ini[0], inq[0], zero);
            P[3] = mfma32(ini[1], inq[1], zero);
            P[4] = mfma32(kcp1, kd0f, zero);
            P[5] = mfma32(kd0f, qcp1, zero);
            floatx4* part = reinterpret_cast<floatx4*>(lds + L::PART + slot * L::PART_SLOT) + p * 6 * 64;
#pragma unroll
            for (int t = 0; t < 6; ++t) part[t * 64 + lane] = P[t];
        };

        // ------------------------------------------------------ compute waves
        // V of chunk x in D layout: element i of block bb is token 16 bb + 4 lg + i
        // (padding tokens re-read a real row: their rows of Tb are zero)
        struct VIn {
            uint32_t w[2][4];
        };
        auto load_v = [&](VIn& d, int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4, lr = m, lg = g;
            (void)lr; (void)lg;
            const int64_t ct0 = chunk_t0(x);
            const uint16_t* vb = a.v + ct0 * vstride + (int64_t)h * V;
            const int nvalid = (int)min((int64_t)C, tseq1 - ct0);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tk = 16 * bb + 4 * lg + i;
                    const int off = (tk < nvalid ? tk * a.H * V : 0) + col_of(0, lr);
                    if constexpr (CT == 2) d.w[bb][i] = *reinterpret_cast<const uint32_t*>(vb + off);
                    else d.w[bb][i] = vb[off];
                }
        };
        // phase B: finish chunk x's record (duty compute wave)
        auto phase_b = [&](int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4, lr = m, lg = g;
            (void)lr; (void)lg;
            const int slot = x & 1;
            unsigned char* rec = lds + L::REC + (x % 3) * R::BYTES;
            const floatx4* part =
                reinterpret_cast<const floatx4*>(lds + L::PART + slot * L::PART_SLOT);
            // the sum of the prep waves' partial products of tile t (fixed order)
            auto tile = [&](int t) __attribute__((always_inline)) {
                floatx4 r = part[t * 64 + lane];
#pragma unroll
                for (int pp = 1; pp < NPW; ++pp) {
                    const floatx4 y = part[(pp * 6 + t) * 64 + lane];
#pragma unroll
                    for (int i = 0; i < 4; ++i) r[i] += y[i];
                }
                return r;
            };
            const float* bs = reinterpret_cast<const float*>(lds + L::BETA) + slot * 32;
            const float* gt = reinterpret_cast<const float*>(lds + L::GTOK) + slot * 32;
            float* am = reinterpret_cast<float*>(lds + L::AMAT);
            floatx4 aq[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const floatx4 pa = tile(b), pq = tile(2 + b);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * g + i;  // row of this element; its column is m
                    const float br = bs[16 * b + r];
                    float dec_rm = 1.f, dec_mr = 1.f;
                    if constexpr (GDN) {
                        const float gr = gt[16 * b + r], gm = gt[16 * b + m];
                        dec_rm = r > m ? exp2_hw(gr - gm) : 0.f;
                        dec_mr = m >= r ? exp2_hw(gm - gr) : 0.f;
                    }
                    am[b * 256 + 16 * r + m] = m < r ? br * pa[i] * dec_rm : 0.f;  // A[r][m]
                    aq[b][i] = r <= m ? pq[i] * dec_mr : 0.f;                     // Aqk[m][r]
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            wave_lds_sync();
            const floatx4 TT0 = tri_inv_row(am, m, g);  // T00[m][4g + i]
            __builtin_amdgcn_sched_barrier(0);
            float* t00 = reinterpret_cast<float*>(lds + L::T00);
            *reinterpret_cast<floatx4*>(t00 + 16 * m + 4 * g) = TT0;
            const floatx4 TT1 = tri_inv_row(am + 256, m, g);  // T11[m][4g + i]
            __builtin_amdgcn_sched_barrier(0);
            wave_lds_sync();
            floatx4 T00D, A10;  // D layout: T00[4g + i][m], A10[4g + i][m]
            const floatx4 p4 = tile(4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                T00D[i] = t00[16 * (4 * g + i) + m];
                A10[i] = bs[16 + 4 * g + i] * p4[i];
            }
            // T10^T = -T00^T A10^T T11^T = -M(T00, M(A10, T11^T))
            const floatx4 T10T = mt(T00D, mt(A10, TT1));
            const floatx4 p5 = tile(5);
            floatx4 tb_lo[2], tb_hi[2], aq_lo[2], aq_hi[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float b0 = bs[4 * g + i], b1 = bs[16 + 4 * g + i];
                tb_lo[0][i] = TT0[i] * b0;    // Tb00
                tb_hi[0][i] = 0.f;
                tb_lo[1][i] = -b0 * T10T[i];  // Tb10
                tb_hi[1][i] = TT1[i] * b1;    // Tb11
                aq_lo[0][i] = aq[0][i];
                aq_hi[0][i] = 0.f;
                aq_lo[1][i] = p5[i];          // Aqk10 (all keys before the query)
                aq_hi[1][i] = aq[1][i];
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                *reinterpret_cast<bf16xEL*>(rec + R::AQK + (b * 64 + lane) * (2 * EL)) =
                    pack_tok(aq_lo[b], aq_hi[b]);
                *reinterpret_cast<bf16xEL*>(rec + R::TB + (b * 64 + lane) * (2 * EL)) =
                    pack_tok(tb_lo[b], tb_hi[b]);
            }
            // the chunk's bound (sum over its tokens of max_c log2 a), warm-up chunks
            if (x < out_from) {
                const float* rm = reinterpret_cast<const float*>(lds + L::RMAX) + slot * NPW * 32;
                float v = -INFINITY;
#pragma unroll
                for (int pp = 0; pp < NPW; ++pp) v = fmaxf(v, rm[pp * 32 + (lane & 31)]);
                // ||I - b k^ k^T||_2 = max(1, |1 - b|) for a unit key (padding: b = 0)
                v += fmaxf(0.f, log2_hw(fabsf(1.f - bs[lane & 31])));
                v = lane < 32 ? v : 0.f;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
                if (lane == 0) misc[0] += v;
            }
        };
        // the recurrence over chunk x (operands from its LDS record)
        auto compute = [&](int x, const VIn& vin) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4, lr = m, lg = g;
            (void)lr; (void)lg;
            const unsigned char* buf = lds + L::REC + (x % 3) * R::BYTES;
            const int64_t ct0 = chunk_t0(x);
            const int nvalid = (int)min((int64_t)C, tseq1 - ct0);
            const bool outs = x >= out_from;
            bf16x8 sb[CT][KS];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int j = 0; j < KS; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sb[ct][j][e] = (bf16)S[ct][2 * j][e];
                        sb[ct][j][4 + e] = (bf16)S[ct][2 * j + 1][e];
                    }
            floatx4 Y[CT][2];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t w = vin.w[bb][i];
                    Y[0][bb][i] = bf_lo(w);
                    if constexpr (CT == 2) Y[1][bb][i] = bf_hi(w);
                }
            // Y_b = V_b - KG_b S
#pragma unroll
            for (int j = 0; j < KS; ++j)
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {
                    const bf16x8 nkg = *reinterpret_cast<const bf16x8*>(
                        buf + R::NKG + ((bb * KS + j) * 64 + lane) * 16);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Y[ct][bb] = mfma32(nkg, sb[ct][j], Y[ct][bb]);
                }
            __builtin_amdgcn_sched_barrier(0);
            // O^T = S^T QG^T (+ U'^T Aqk^T below)
            floatx4 OT[CT][2];
            const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
            if (outs) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int ob = 0; ob < 2; ++ob) OT[ct][ob] = zero;
#pragma unroll
                for (int j = 0; j < KS; ++j)
#pragma unroll
                    for (int ob = 0; ob < 2; ++ob) {
                        const bf16x8 qg = *reinterpret_cast<const bf16x8*>(
                            buf + R::QG + ((ob * KS + j) * 64 + lane) * 16);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) OT[ct][ob] = mfma32(sb[ct][j], qg, OT[ct][ob]);
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
            // decay the state
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const floatx4 gc =
                    *reinterpret_cast<const floatx4*>(buf + R::GAMC + (16 * t + 4 * lg) * 4);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[ct][t][i] *= gc[i];
            }
            __builtin_amdgcn_sched_barrier(0);
            // U' = Tb Y over the chunk's tokens
            bf16xEL yc[CT], uc[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    yc[ct][i] = (bf16)Y[ct][0][i];
                    yc[ct][4 + i] = (bf16)Y[ct][1][i];
                }
            floatx4 U[CT][2];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const bf16xEL tb =
                    *reinterpret_cast<const bf16xEL*>(buf + R::TB + (bb * 64 + lane) * (2 * EL));
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) U[ct][bb] = mfma_tok(tb, yc[ct], zero);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uc[ct][i] = (bf16)U[ct][0][i];
                    uc[ct][4 + i] = (bf16)U[ct][1][i];
                }
            __builtin_amdgcn_sched_barrier(0);
            // S = Diag(Gam_C) S + KdT U'
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const bf16xEL kdt = *reinterpret_cast<const bf16xEL*>(
                    buf + R::KDT + st_unit(t * 64 + lane) * 16);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) S[ct][t] = mfma_tok(kdt, uc[ct], S[ct][t]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (!outs) return;
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                const bf16xEL aqk =
                    *reinterpret_cast<const bf16xEL*>(buf + R::AQK + (ob * 64 + lane) * (2 * EL));
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) OT[ct][ob] = mfma_tok(uc[ct], aqk, OT[ct][ob]);
            }
            // OT[ct][ob][i] = O[token 16 ob + lr][column of tile ct, tile row 4 lg + i]
            uint16_t* obase = a.o + ct0 * vstride + (int64_t)h * V;
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                if (16 * ob + lr >= nvalid) continue;
                uint16_t* op = obase + (16 * ob + lr) * a.H * V;
                if constexpr (CT == 2) {
                    // tile ct row 4 lg + i is column wcol + 2 (4 lg + i) + ct: the
                    // lane's 8 values are columns wcol + 8 lg .. + 7
                    bf16x8 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ov[2 * i] = (bf16)(a.scale * OT[0][ob][i]);
                        ov[2 * i + 1] = (bf16)(a.scale * OT[1][ob][i]);
                    }
                    *reinterpret_cast<bf16x8*>(op + wcol + 8 * lg) = ov;
                } else {
                    bf16x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov[i] = (bf16)(a.scale * OT[0][ob][i]);
                    *reinterpret_cast<bf16x4*>(op + wcol + 4 * lg) = ov;
                }
            }
        };

    // ------------------------------------------------------- the iterations
    // Iteration it (from -4): compute chunk it, phase B chunk it+1, phase A
    // chunk it+2, phase N chunk it+3, loads chunk it+4.  Each role runs its own
    // copy of the loop (the same iterations and barriers), unrolled by three so
    // that every register ring slot is a constant.
    if (is_cw) {
        for (int attempt = 0; attempt < 2; ++attempt) {
            begin_attempt(attempt);
            load_state(exact);
            if (tid == 0) misc[0] = 0.f;  // sum of the warm-up chunks' bounds
            if (n_it <= 0) break;
            const int n_iter = (n_it + 4 + 2) / 3 * 3;
            VIn vin[3];
            bool restart = false;
            for (int k3 = 0; k3 < n_iter && !restart; k3 += 3) {
                static_for<0, 3>([&](auto u) __attribute__((always_inline)) {
                    if (restart) return;
                    const int it = k3 + u - 4;
                    if (failed_bound(it)) {
                        restart = true;
                        return;
                    }
                    constexpr int sv = (u + 1) % 3, sc = (u + 2) % 3;
                    // unconditional (a valid chunk re-read at the ends): a load
                    // issued on some paths only makes the compiler's in-order
                    // wait counts cover the loads just issued as well
                    load_v(vin[sv], min(max(it + 2, 0), n_it - 1));
                    if (it + 1 >= 0 && it + 1 < n_it && wave == (it + 1) % NCW) phase_b(it + 1);
                    if (it >= 0 && it < n_it) compute(it, vin[sc]);
                    __syncthreads();
                });
            }
            if (!restart) break;
            __syncthreads();  // every wave has read the bound before it is reset
        }
        if (fslot >= 0 && a.final_state) {
            const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4;
            float* fp = a.final_state + ((int64_t)fslot * a.H + h) * K * V;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        fp[tile_channel(t, 4 * lg + i) * V + col_of(ct, lr)] = S[ct][t][i];
        }
    } else {
        for (int attempt = 0; attempt < 2; ++attempt) {
            begin_attempt(attempt);
            if (n_it <= 0) break;
            const int n_iter = (n_it + 4 + 2) / 3 * 3;
            // nothing in flight on entry (a restarted attempt leaves loads of
            // the abandoned one): the loop's wait counts hold on every path
            __builtin_amdgcn_s_waitcnt(VMCNT_0);
            PIn pin[3];
            bool restart = false;
            for (int k3 = 0; k3 < n_iter && !restart; k3 += 3) {
                static_for<0, 3>([&](auto u) __attribute__((always_inline)) {
                    if (restart) return;
                    const int it = k3 + u - 4;
                    if (failed_bound(it)) {
                        restart = true;
                        return;
                    }
                    constexpr int sl = u, sn = (u + 2) % 3, sa = (u + 1) % 3;
                    load_in(pin[sl], min(it + 4, n_it - 1));  // unconditional (see load_v)
                    if (it + 3 >= 0 && it + 3 < n_it) phase_n(pin[sn], it + 3);
                    if (it + 2 >= 0 && it + 2 < n_it) phase_a(pin[sa], it + 2);
                    else touch(pin[sa]);
                    __syncthreads();
                });
            }
            if (!restart) break;
            __syncthreads();
        }
    }
}

template <int K, int V, bool GDN>
static void launch_fused_t(const FusedArgs& a, int n_groups, hipStream_t stream,
                           const LaunchEvents* ev) {
    using Lay = FusedLayout<K, V>;
    const dim3 grid((unsigned)n_groups), block(Lay::NT);
    if (ev)
        hipExtLaunchKernelGGL((kda_fused_kernel<K, V, GDN>), grid, block, 0, stream, ev->start,
                              ev->stop, 0, a);
    else
        hipLaunchKernelGGL((kda_fused_kernel<K, V, GDN>), grid, block, 0, stream, a);
}

void launch_fused(const FusedArgs& a, int K, int V, bool gdn, int n_groups, hipStream_t stream,
                  const LaunchEvents* ev) {
    if (n_groups <= 0) return;
    if (K == 128) {
        if (V == 128) gdn ? launch_fused_t<128, 128, true>(a, n_groups, stream, ev)
                          : launch_fused_t<128, 128, false>(a, n_groups, stream, ev);
        else gdn ? launch_fused_t<128, 64, true>(a, n_groups, stream, ev)
                 : launch_fused_t<128, 64, false>(a, n_groups, stream, ev);
    } else {
        if (V == 128) gdn ? launch_fused_t<64, 128, true>(a, n_groups, stream, ev)
                          : launch_fused_t<64, 128, false>(a, n_groups, stream, ev);
        else gdn ? launch_fused_t<64, 64, true>(a, n_groups, stream, ev)
                 : launch_fused_t<64, 64, false>(a, n_groups, stream, ev);
    }
}

}  // namespace kda
