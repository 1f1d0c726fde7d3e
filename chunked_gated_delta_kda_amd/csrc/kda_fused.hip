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
//     chunk, over two iterations: load q, k, g (and beta); then (phase A) the
//     gate, the in-block prefix sums, the decayed operands written into the
//     chunk's LDS record, partial intra-chunk products over its channels and
//     partial squared norms of q and k (diagonals of MFMA products of the raw
//     inputs).  q and k are never normalised elementwise: the record holds
//     the raw rows and the per-token factors 1/||k||, 1/||q|| are applied to
//     the 16x16 tiles, to V - KG S, to U' and to the output.
//   compute waves (4): wave w owns V/4 value columns of the [K, V] state in
//     fp32 MFMA accumulators for the whole segment and runs the recurrence of
//     kda_recur.hip on the LDS record.  Each of them also finishes a quarter
//     of the next chunk's record (phase B, in four parts that rotate over the
//     waves): two parts form a block's A (sums of the prep waves' partial
//     products, beta, norms), its inverse and Tb; the other two the norms,
//     the Aqk tiles and the decay bound.  The coupling block
//     Tb10 = -(T11 A10) Tb00 is formed by every compute wave at its next
//     step from fp32 tiles the two inverse parts left in LDS.
//   phase-B waves (4, scalar gate only): the scalar gate's phase A is light
//     and its compute waves, carrying phase B too, set the pace; with phase B
//     on four waves of its own (same parts, same rotation) each SIMD runs
//     three waves at up to 168 registers each.  To fit, the scalar gate's
//     recurrence forms S's bf16 operand one 32-channel slice at a time and
//     its prep waves issue each block's partial products as soon as that
//     block's operands exist, and the coupling block Tb10 is formed once, by
//     the wave of part 2 after parts 0 and 1 signal through LDS flags, and
//     read from the record by the compute waves.  (The per-channel gate, whose prep waves are as
//     long as its compute waves, measured 10% slower with the third wave: at
//     168 registers its prep waves no longer keep their loads in flight
//     across the decayed products.)
// One barrier per iteration.  In iteration i the compute waves run chunk i,
// phase B finishes chunk i+1 and phase A fills chunk i+2; three records are
// live in LDS.
//
// Sequence segments.  A (sequence, head) pair is one chain of chunk steps, so
// long sequences are cut into segments of L chunks that run in parallel.  A
// segment that does not start its sequence starts its recurrence from a zero
// state W chunks early (the warm-up) and checks the bound of those chunks'
// transitions: for one token ||(I - b k^ k^T) Diag(a)||_2 <= max(1, |1 - b|)
// max_c a_c (at most max_c a_c for 0 <= b <= 2), so the state entering the
// segment reaches its first token scaled by at most 2^(the sum over the
// warm-up's tokens of log2 of that factor).  Below 2^bound_limit (2^-24: the
// fp32 rounding of the state) the zero start is exact to that bound.
// Otherwise the segment tries again with a longer warm-up, and if that
// fails too, from the sequence start and its initial state.  The bound is
// known when the warm-up ends, so a failed attempt costs only its warm-up
// and the pipeline's two fill iterations.  The FlashQLA summary (section "핵심 기능") describes switching on
// intra-card parallelism when the gate's decay allows it; this is that test,
// made per segment.
#include <hip/hip_ext.h>

#include "kda_common.h"
#include "kda_launch.h"
#include "kda_ops.h"

namespace kda {

namespace {

template <int K, int V, bool GDN>
struct FusedLayout {
    using R = Rec<K>;
    static constexpr int NPW = K / 32;  // prep waves
    static constexpr int NCW = 4;       // compute waves
    // phase-B waves: the scalar gate runs phase B on waves of its own (three
    // waves per SIMD); the per-channel gate on the compute waves
    static constexpr int NBW = GDN ? NCW : 0;
    static constexpr int CT = V / 64;   // 16-column state tiles per compute wave
    static constexpr int NT = 64 * (NPW + NCW + NBW);
    static constexpr int NBUF = 3;      // chunk records in LDS
    // byte offsets: the small tables and the partial products first, so that
    // every access to them is a lane offset plus an instruction immediate
    // (LDS instructions encode offsets below 64 KB); the records last (their
    // accesses start from a per-record base anyway)
    static constexpr int NRM = 0;                                   // [2][NPW][64] float
    static constexpr int RMAX = NRM + 2 * NPW * 64 * 4;             // [2][NPW][32] float
    static constexpr int BETA = RMAX + 2 * NPW * 32 * 4;            // [2][32] float
    static constexpr int GTOK = BETA + 2 * 32 * 4;                  // [2][32] float
    static constexpr int AMAT = GTOK + 2 * 32 * 4;                  // [2][256] float
    // [2][2][256] float: per chunk (slot x & 1) Tb00 row-major and
    // (T11 A10)^T in D layout, from phase B for the coupling block the
    // compute waves form
    static constexpr int CPL = AMAT + 2 * 256 * 4;
    static constexpr int INVN = CPL + 2 * 2 * 256 * 4;              // [NBUF][64] float
    static constexpr int MISC = INVN + NBUF * 64 * 4;               // bound sum
    static constexpr int PART = MISC + 16;                          // [2][NPW][6][64] floatx4
    static constexpr int PART_SLOT = NPW * 6 * 64 * 16;
    static constexpr int REC = PART + 2 * PART_SLOT;                // [NBUF][R::BYTES]
    static constexpr int BYTES = REC + NBUF * R::BYTES;
    static_assert(PART % 16 == 0 && REC % 16 == 0, "16-byte LDS accesses");
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
// length.  The compute waves use it (hoisting there took them from 222 to
// 237 VGPRs and measured 3-5% slower); the prep waves, well below the
// kernel's register count, use the plain lane index and keep those values.
__device__ __forceinline__ int opaque_lane() {
    int l = (int)(threadIdx.x & 63);
    asm volatile("" : "+v"(l));
    return l;
}

// A wave-uniform value the compiler cannot see through: record and slot
// indices derived from the chunk number stay plain products, instead of
// being strength-reduced into loop-carried addresses whose displacements
// (negative) no LDS instruction can encode, which costs an add per access.
__device__ __forceinline__ int opaque_uniform(int v) {
    asm volatile("" : "+s"(v));
    return v;
}

// s_waitcnt immediates that wait until at most eight (none) vector memory
// loads are outstanding (vmcnt 8 / 0; expcnt and lgkmcnt left at their maximum)
constexpr int VMCNT_8 = 0x0F78;
constexpr int VMCNT_0 = 0x0F70;

// element i (runtime, 0..3) of v
__device__ __forceinline__ float pick(floatx4 v, int i) {
    const float lo = i & 1 ? v[1] : v[0], hi = i & 1 ? v[3] : v[2];
    return i & 2 ? hi : lo;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// lane 15 of each 16-lane row, broadcast to the row (ds_swizzle bit mode:
// and 0x10, or 0x0f within each half of the wave)
__device__ __forceinline__ float row_last(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1f0));
}

// An LDS flag set by one wave and awaited by another within an iteration
// (bounded: a wait that runs out proceeds, so no path can hang).
__device__ __forceinline__ void flag_set(int* f, int v) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void flag_wait(int* f, int v) {
    for (int n = 0; n < (1 << 22); ++n) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == v) break;
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace

// STORE (KDA, two column tiles a wave): the variant that also keeps, for
// every chunk with outputs, the bf16 state entering it and its V - KG S (the
// quantities the backward pass reads), with the outputs optional (a.o may be
// null).  GDN's twelve waves have 168 registers each, too few for the stores
// without spilling.
template <int K, int V, bool GDN, bool STORE>
__global__ __launch_bounds__(64 * (K / 32 + (GDN ? 8 : 4))) void kda_fused_kernel(FusedArgs a) {
    using L = FusedLayout<K, V, GDN>;
    using R = Rec<K>;
    constexpr int NPW = L::NPW, NCW = L::NCW, NBW = L::NBW, CT = L::CT;
    constexpr int KS = K / 32, KT = K / 16;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::BYTES];

    // ---------------------------------------------------------------- segment
    const int h = blockIdx.x % a.H;
    int vseg = blockIdx.x / a.H;
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
        // dispatch rank -> segment (longest first), kept inside the table
        if (a.order) vseg = min(max(a.order[vseg], 0), nseg - 1);
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
    const bool is_bw = NBW > 0 && wave >= NCW && wave < NCW + NBW;
    const int p = wave - NCW - NBW;  // prep wave index (>= 0 for prep waves)

    // ---------------------------------------------------- compute-wave state
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
            if constexpr (CT == 2) {
                // the two tiles' columns 2 lr and 2 lr + 1 are adjacent: one
                // 8-byte load per (tile row, channel)
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float2 v = *reinterpret_cast<const float2*>(
                            sp + tile_channel(t, 4 * lg + i) * V + col_of(0, lr));
                        S[0][t][i] = v.x;
                        S[1][t][i] = v.y;
                    }
            } else {
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[0][t][i] = sp[tile_channel(t, 4 * lg + i) * V + col_of(0, lr)];
            }
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
        if (p >= 0) {
            const float* dp = a.dt_bias + (int64_t)h * K + 32 * p + 8 * g;
#pragma unroll
            for (int e = 0; e < 8; ++e) dt[e] = dp[e] * LOG2E;  // the gate works in log2 units
        }
    }

    float* const misc = reinterpret_cast<float*>(lds + L::MISC);
    int* const flags = reinterpret_cast<int*>(lds + L::MISC) + 1;  // [2]: parts 0, 1 done (phase-B waves)

    // An attempt computes chunks x0 .. c1 - 1 of the sequence, with outputs
    // from c0 on; attempts 0 and 1 (each after a failed bound) start
    // warm_chunks and warm_chunks_retry chunks early from a zero state (exact
    // when that is the sequence start), attempt 2 from the sequence start and
    // its initial state.
    constexpr int N_ATTEMPTS = 3;
    int x0 = 0, n_it = 0, out_from = 0;
    bool exact = true;
    // the attempt's first (token, head) row and its tokens up to the sequence
    // end: per chunk, a 32-bit token offset from there (the batch holds fewer
    // than 2^31 tokens)
    int64_t row0 = 0;
    int seg_len = 0;
    auto begin_attempt = [&](int attempt) __attribute__((always_inline)) {
        const int w = attempt == 0 ? a.warm_chunks : attempt == 1 ? a.warm_chunks_retry : c0;
        x0 = max(0, c0 - w);                     // first chunk computed
        exact = x0 == 0;
        n_it = c1 - x0;                          // chunks computed
        out_from = c0 - x0;                      // first chunk (relative) with outputs
        const int64_t t0 = tseq0 + (int64_t)C * x0;
        row0 = t0 * a.H + h;
        seg_len = (int)(tseq1 - t0);
    };
    // the warm-up chunks' bound is complete at iteration out_from (phase B of
    // the last one ran an iteration earlier); every wave reads the same value
    auto failed_bound = [&](int it) __attribute__((always_inline)) {
        if (exact || it != out_from) return false;
        // the LDS read stays here (not hoisted into every iteration)
        asm volatile("" ::: "memory");
        return !(misc[0] < a.bound_limit);
    };

        // ---------------------------------------------------------- prep waves
        // chunk x (relative to x0): its valid tokens, and the byte offset of its
        // first row from the attempt's first row, for rows of `row_bytes`
        auto nvalid_of = [&](int x) __attribute__((always_inline)) { return min(C, seg_len - C * x); };
        auto chunk_off = [&](int x, uint32_t row_bytes) __attribute__((always_inline)) {
            return (uint64_t)(uint32_t)(C * x * a.H) * row_bytes;
        };
        auto load_in = [&](PIn& d, int x) __attribute__((always_inline)) {
            const int lane = (int)(threadIdx.x & 63), m = lane & 15, g = lane >> 4, lr = m, lg = g;
            (void)lr; (void)lg;
            // uniform bases and 32-bit lane byte offsets (one address add per load)
            const uint64_t ok = chunk_off(x, 2u * K), o2 = chunk_off(x, 2u), o4 = chunk_off(x, 4u);
            const char* qb = reinterpret_cast<const char*>(a.q + row0 * K) + ok;
            const char* kb = reinterpret_cast<const char*>(a.k + row0 * K) + ok;
            const char* gb = GDN ? nullptr : reinterpret_cast<const char*>(a.g_kda + row0 * K) + ok;
            const char* gdb = GDN ? reinterpret_cast<const char*>(a.g_gdn + row0) + o4 : nullptr;
            const char* bt = reinterpret_cast<const char*>(a.beta + row0) + o2;
            (void)o4;
            const int nvalid = nvalid_of(x);
            const uint32_t cb = 32 * p + 8 * g;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                // padding rows re-read the chunk's first row
                const uint32_t r = 16 * b + m < nvalid ? (uint32_t)(16 * b + m) * (uint32_t)a.H : 0u;
                const uint32_t off = (r * K + cb) * 2u;
                d.q[b] = *reinterpret_cast<const u32x4*>(qb + off);
                d.k[b] = *reinterpret_cast<const u32x4*>(kb + off);
                if constexpr (!GDN) d.g[b] = *reinterpret_cast<const u32x4*>(gb + off);
                else d.gd[b] = *reinterpret_cast<const float*>(gdb + r * 4u);
                d.braw[b] = *reinterpret_cast<const uint16_t*>(bt + r * 2u);
            }
        };
        // `issue_loads` runs between the decay scan and the rest: the next
        // chunks' loads leave the wave after its first long run of arithmetic,
        // not at the barrier where every wave of the CU issues at once
        auto phase_a = [&](const PIn& d, int x, auto&& issue_loads) __attribute__((always_inline)) {
            const int lane = (int)(threadIdx.x & 63), m = lane & 15, g = lane >> 4, lr = m, lg = g;
            (void)lr; (void)lg;
            const int slot = opaque_uniform(x & 1);
            unsigned char* rec = lds + L::REC + opaque_uniform(x % 3) * R::BYTES;
            const int nvalid = nvalid_of(x);
            float vmask[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) vmask[b] = 16 * b + m < nvalid ? 1.f : 0.f;
            if (p == 0) {  // beta of the chunk's tokens (one prep wave)
                float bsig[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const float braw = __uint_as_float((uint32_t)d.braw[b] << 16);
                    bsig[b] = vmask[b] > 0.f ? (GDN ? braw : sigmoid_f(braw)) : 0.f;
                }
                if (g == 0) {
                    float* bs = reinterpret_cast<float*>(lds + L::BETA) + slot * 32;
                    bs[m] = bsig[0];
                    bs[16 + m] = bsig[1];
                }
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
                    // with y' = (g + dt_bias) log2 e:
                    // log2 a = max(lb log2 e, -rate log2(1 + 2^y')).  Where 2^y'
                    // overflows the product is -inf (the floor binds), or NaN
                    // for a padding row (factor -0), which the max drops (IEEE
                    // maxNum returns the number): padding rows get 0
                    const float lb2 = a.lower_bound * LOG2E * vmask[b];
                    const float c1v = -rate * vmask[b];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float x2[2] = {bf_lo(d.g[b][u]), bf_hi(d.g[b][u])};
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int e = 2 * u + hh;
                            const float y = fmaf(x2[hh], LOG2E, dt[e]);
                            G[b][e] = fmaxf(lb2, c1v * log2_hw(1.f + exp2_hw(y)));
                        }
                    }
                }
                row_scan16_n<16>(&G[0][0]);
                // the scan's results used here: later uses inside lane-masked
                // blocks would otherwise pull its last step there, unfused
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(G[b][e]));
            }
            issue_loads();
            if (x < out_from) {  // only warm-up chunks need the bound
                if constexpr (!GDN) {
                    // the bound: max over this wave's channels of each token's
                    // log2 decay (the differences of the prefix sums; the row's
                    // first lane reads 0), then over the lane's row groups
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        rmax[b] = -INFINITY;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float prev =
                                __builtin_amdgcn_update_dpp(0.f, G[b][e], ROW_SHR1, 0xf, 0xf, true);
                            rmax[b] = fmaxf(rmax[b], G[b][e] - prev);
                        }
                    }
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
            }
            // per-channel block decays 2^(block total): ef0 (block 0), ef1 (block 1)
            float ef0[8], ef1[8];
            float glk[2][8];  // KDA: 2^G, the decay from the block start
            (void)glk;
            if constexpr (GDN) {
                const float t0 = row_last(Gs[0]), t1 = row_last(Gs[1]);
                const float e0 = exp2_hw(t0), e1 = exp2_hw(t1);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ef0[e] = e0;
                    ef1[e] = e1;
                }
            } else {
                // the block totals' decays are 2^G of the block's last row
                // (padding rows add nothing): broadcast from lane 15 of the row
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 8; ++e) glk[b][e] = exp2_hw(G[b][e]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ef0[e] = row_last(glk[0][e]);
                    ef1[e] = row_last(glk[1][e]);
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
                    qn[2 * u] = bf_lo(d.q[b][u]);
                    qn[2 * u + 1] = bf_hi(d.q[b][u]);
                    kn[2 * u] = bf_lo(d.k[b][u]);
                    kn[2 * u + 1] = bf_hi(d.k[b][u]);
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
                        gl = glk[b][e];
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
                // KG itself in the record's nKG slot: the recurrence negates it in
                // the FMA that adds V (a source modifier, no instruction)
                *reinterpret_cast<bf16x8*>(rec + R::NKG + ((b * KS + p) * 64 + lane) * 16) = pack8(kg);
                *reinterpret_cast<bf16x8*>(rec + R::QG + ((b * KS + p) * 64 + lane) * 16) = pack8(qg);
                // KdT[t][g'][m'][e'] = Kd[tok(g', e')][rho(t, m')], 16-byte units
                // swizzled by st_unit.  Channel 32p + 8g + e is row 4g + (e & 3) of
                // tile t = 2p + (e >> 2) and token m (block b) is element 4b + (m & 3)
                // of unit 16 (4t + (m >> 2)) + row; st_unit XORs (m >> 2) & 3 into
                // the row's low bits, so the element index is
                //   1024 p + 128 (m >> 2) + 32 g + (m & 3) + 8 ((e & 3) ^ ((m >> 2) & 3))
                //   + 512 (e >> 2) + 4 b:
                // four lane addresses (one per e & 3) and constant offsets.
                {
                    const u32x4 w = __builtin_bit_cast(u32x4, pack8(kd));
                    const int lb = 1024 * p + 128 * (m >> 2) + 32 * g + (m & 3), sw = (m >> 2) & 3;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        uint16_t* kp = kdt + lb + 8 * ((e & 3) ^ sw);
                        kp[512 * (e >> 2) + 4 * b] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
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
                // With phase-B waves (168 registers a wave) this block's
                // partial products over the wave's 32 channels (D = X Y^T) and
                // its rows' squared norms, as soon as its operands exist (the
                // block's operands then die early); otherwise all at the end,
                // below:
                //   0: A00 (in-block K Ki^T)  1: A11  2: Aqk00^T (Ki Q^T)  3: Aqk11^T
                //   4: A10 (KG1 Kd0^T)        5: Aqk10^T (Kd0 QG1^T)
                if constexpr (NBW > 0) {
                    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
                    floatx4* part = reinterpret_cast<floatx4*>(lds + L::PART + slot * L::PART_SLOT) + p * 6 * 64;
                    part[b * 64 + lane] = mfma32(ink[b], ini[b], zero);
                    part[(2 + b) * 64 + lane] = mfma32(ini[b], inq[b], zero);
                    if (b == 1) {
                        part[4 * 64 + lane] = mfma32(kcp1, kd0f, zero);
                        part[5 * 64 + lane] = mfma32(kd0f, qcp1, zero);
                    }
                    // squared norms of the raw rows: diagonals of Q Q^T and K K^T
                    float* nr = reinterpret_cast<float*>(lds + L::NRM) + (slot * NPW + p) * 64;
                    const bf16x8 kr = __builtin_bit_cast(bf16x8, d.k[b]);
                    const bf16x8 qr = __builtin_bit_cast(bf16x8, d.q[b]);
                    const floatx4 dk = mfma32(kr, kr, zero), dq = mfma32(qr, qr, zero);
                    if (g == (m >> 2)) {
                        nr[16 * b + m] = pick(dk, m & 3);
                        nr[32 + 16 * b + m] = pick(dq, m & 3);
                    }
                }
            }
            if constexpr (NBW > 0) return;
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
            // Squared norms of the raw q and k rows over this wave's channels:
            // the diagonals of Q Q^T and K K^T from the bf16 inputs (exact
            // products, fp32 sums).  q and k stay unnormalised everywhere above;
            // phase B and the recurrence apply 1/||k|| and 1/||q|| per token.
            float* nr = reinterpret_cast<float*>(lds + L::NRM) + (slot * NPW + p) * 64;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const bf16x8 kr = __builtin_bit_cast(bf16x8, d.k[b]);
                const bf16x8 qr = __builtin_bit_cast(bf16x8, d.q[b]);
                const floatx4 dk = mfma32(kr, kr, zero), dq = mfma32(qr, qr, zero);
                // D[4 g + i][m]: the diagonal is in the lanes of g = m >> 2, element m & 3
                if (g == (m >> 2)) {
                    nr[16 * b + m] = pick(dk, m & 3);
                    nr[32 + 16 * b + m] = pick(dq, m & 3);
                }
            }
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
            const char* vb = reinterpret_cast<const char*>(a.v + row0 * V) + chunk_off(x, 2u * V);
            const int nvalid = nvalid_of(x);
            const uint32_t rstride = (uint32_t)a.H * V;
            if (nvalid == C) {
                // a whole chunk: one lane offset, the rows' bases wave-uniform
                const uint32_t off = ((uint32_t)(4 * lg) * rstride + (uint32_t)col_of(0, lr)) * 2u;
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const char* rb = vb + (size_t)((16 * bb + i) * rstride) * 2u;
                        if constexpr (CT == 2) d.w[bb][i] = *reinterpret_cast<const uint32_t*>(rb + off);
                        else d.w[bb][i] = *reinterpret_cast<const uint16_t*>(rb + off);
                    }
                return;
            }
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tk = 16 * bb + 4 * lg + i;
                    const uint32_t off =
                        ((tk < nvalid ? (uint32_t)tk * rstride : 0u) + (uint32_t)col_of(0, lr)) * 2u;
                    if constexpr (CT == 2) d.w[bb][i] = *reinterpret_cast<const uint32_t*>(vb + off);
                    else d.w[bb][i] = *reinterpret_cast<const uint16_t*>(vb + off);
                }
        };
        // phase B: finish chunk x's record in four parts, one per compute wave,
        // that run at the same time: P0 block 0 (A00, T00, Tb00), P1 block 1
        // (A11, T11, Tb11, the coupling tile A10 and the product T11 A10), P2
        // the chunk's norms and Aqk00, P3 Aqk11, Aqk10 and the decay bound.
        // The two substitutions, the long chains, sit on SIMDs two apart; the
        // light parts keep them free of everything else.  The coupling block
        // Tb10 = -(T11 A10) Tb00 of Tb is left to the compute waves (from the
        // fp32 tiles in CPL: P0's and P1's results meet only there).
        // The sum of the prep waves' partial products of tile t (fixed order):
        auto tile = [&](int slot, int t, int lane) __attribute__((always_inline)) {
            const floatx4* part =
                reinterpret_cast<const floatx4*>(lds + L::PART + slot * L::PART_SLOT);
            floatx4 r = part[t * 64 + lane];
#pragma unroll
            for (int pp = 1; pp < NPW; ++pp) {
                const floatx4 y = part[(pp * 6 + t) * 64 + lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] += y[i];
            }
            return r;
        };
        // 1/||k|| of chunk token s (lane-varying) and of block b's rows
        // 4 g + i, from the prep waves' partial squared norms; 0 for padding
        auto token_norm = [&](int slot, int s, int nvalid) __attribute__((always_inline)) {
            const float* nr = reinterpret_cast<const float*>(lds + L::NRM) + slot * NPW * 64;
            float v = nr[s];
#pragma unroll
            for (int pp = 1; pp < NPW; ++pp) v += nr[pp * 64 + s];
            return s < nvalid ? rsq_hw(v + NORM_EPS) : 0.f;
        };
        auto row_norms = [&](int slot, int b, int nvalid, int g) __attribute__((always_inline)) {
            const float* nr = reinterpret_cast<const float*>(lds + L::NRM) + slot * NPW * 64;
            floatx4 ikr = *reinterpret_cast<const floatx4*>(nr + 16 * b + 4 * g);
#pragma unroll
            for (int pp = 1; pp < NPW; ++pp) {
                const floatx4 y = *reinterpret_cast<const floatx4*>(nr + pp * 64 + 16 * b + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) ikr[i] += y[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ikr[i] = 16 * b + 4 * g + i < nvalid ? rsq_hw(ikr[i] + NORM_EPS) : 0.f;
            return ikr;
        };
        // A[r][m] of block b (r = 4 g + i) into am (row-major) and ad (D
        // layout): beta_r k^_r . k^_m from the raw-key partials, decay-weighted
        // for GDN
        auto build_a = [&](int slot, int b, const floatx4& pa, const floatx4& ikr, float ikm,
                           float* am, int m, int g, floatx4& ad) __attribute__((always_inline)) {
            const float* bs = reinterpret_cast<const float*>(lds + L::BETA) + slot * 32;
            const float* gt = reinterpret_cast<const float*>(lds + L::GTOK) + slot * 32;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;  // row of this element; its column is m
                const float br = bs[16 * b + r] * ikr[i] * ikm;
                if constexpr (GDN) {
                    // formed before the mask: used on one side of the select,
                    // the decay's exp is otherwise sunk into a branch per
                    // element, each waiting on its own LDS reads
                    float v = br * pa[i] * exp2_hw(gt[16 * b + r] - gt[16 * b + m]);
                    asm volatile("" : "+v"(v));
                    ad[i] = m < r ? v : 0.f;
                } else {
                    ad[i] = m < r ? br * pa[i] : 0.f;
                }
                am[16 * r + m] = ad[i];
            }
        };
        // Aqk[m][r] of block b (raw q . k; the norms are applied by the
        // recurrence), decay-weighted for GDN
        auto build_aq = [&](int slot, int b, const floatx4& pq, int m, int g)
            __attribute__((always_inline)) {
            const float* gt = reinterpret_cast<const float*>(lds + L::GTOK) + slot * 32;
            floatx4 aq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                float dec = 1.f;
                if constexpr (GDN) dec = m >= r ? exp2_hw(gt[16 * b + m] - gt[16 * b + r]) : 0.f;
                aq[i] = r <= m ? pq[i] * dec : 0.f;
            }
            return aq;
        };
        // T^T of a block in D layout (T^T[4g + i][m] = T[m][4g + i]) from A in
        // D layout (ad) and row-major in LDS (am, written and synchronised):
        // KDA by fp32 forward substitution on the VALU; GDN, whose phase B
        // and recurrence step are the iteration's critical path (its prep
        // waves' elementwise work is light), by the fp32 doubling product on
        // the otherwise idle MFMA unit.
        // T^T of a block in D layout (T^T[4g + i][m] = T[m][4g + i]) from A in
        // D layout (ad) and row-major in LDS (am, written and synchronised;
        // overwritten here): the two 8 x 8 diagonal blocks by substitution on
        // the VALU, the coupling of the two on fp32 MFMA (28 fmas and eight
        // MFMAs per lane instead of the 16 x 16 substitution's 120 fmas; the
        // iteration is bound by the SIMDs' issue, not by MFMA latency)
        auto block_inverse_t = [&](const floatx4& ad, float* am, int m, int g)
            __attribute__((always_inline)) { return tri_inv_split_t(am, ad, m, g); };
        // Phase B, part 0: block 0's A00, T00 and Tb00
        auto phase_p0 = [&](int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4;
            const int slot = opaque_uniform(x & 1);
            unsigned char* rec = lds + L::REC + opaque_uniform(x % 3) * R::BYTES;
            const float* bs = reinterpret_cast<const float*>(lds + L::BETA) + slot * 32;
            float* am = reinterpret_cast<float*>(lds + L::AMAT);
            const int nvalid = nvalid_of(x);
            const floatx4 ikr = row_norms(slot, 0, nvalid, g);
            const float ikm = token_norm(slot, m, nvalid);
            const floatx4 pa = tile(slot, 0, lane);
            floatx4 ad;
            build_a(slot, 0, pa, ikr, ikm, am, m, g, ad);
            wave_lds_sync();
            const floatx4 TT0 = block_inverse_t(ad, am, m, g);  // T00[m][4g + i]
            floatx4 tb;
#pragma unroll
            for (int i = 0; i < 4; ++i) tb[i] = TT0[i] * bs[4 * g + i];  // Tb00[m][4g + i]
            const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<bf16xEL*>(rec + R::TB + lane * (2 * EL)) = pack_tok(tb, zero);
            float* cpl = reinterpret_cast<float*>(lds + L::CPL) + slot * 512;
            *reinterpret_cast<floatx4*>(cpl + 16 * m + 4 * g) = tb;  // Tb00 row-major
            if constexpr (NBW > 0) flag_set(flags, x + 1);
        };
        // Phase B, part 1: block 1's A11, T11, Tb11 and the product T11 A10
        auto phase_p1 = [&](int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4;
            const int slot = opaque_uniform(x & 1);
            unsigned char* rec = lds + L::REC + opaque_uniform(x % 3) * R::BYTES;
            const float* bs = reinterpret_cast<const float*>(lds + L::BETA) + slot * 32;
            float* am = reinterpret_cast<float*>(lds + L::AMAT) + 256;
            const int nvalid = nvalid_of(x);
            const floatx4 ikr = row_norms(slot, 1, nvalid, g);
            const float ikm1 = token_norm(slot, 16 + m, nvalid), ikm0 = token_norm(slot, m, nvalid);
            const floatx4 pa = tile(slot, 1, lane), p4 = tile(slot, 4, lane);
            floatx4 ad;
            build_a(slot, 1, pa, ikr, ikm1, am, m, g, ad);
            floatx4 a10;  // A10[4g + i][m] = beta_{16+4g+i} k^_{16+4g+i} . k^_m
#pragma unroll
            for (int i = 0; i < 4; ++i) a10[i] = bs[16 + 4 * g + i] * ikr[i] * ikm0 * p4[i];
            wave_lds_sync();
            const floatx4 TT1 = block_inverse_t(ad, am, m, g);  // T11[m][4g + i]
            bf16x4 tb11;
#pragma unroll
            for (int i = 0; i < 4; ++i) tb11[i] = (bf16)(TT1[i] * bs[16 + 4 * g + i]);
            // Tb block 1 = [Tb10 | Tb11]: the Tb11 half here
            *reinterpret_cast<bf16x4*>(rec + R::TB + (64 + lane) * (2 * EL) + EL) = tb11;
            // M(A10, T11^T) = (T11 A10)^T in D layout: once here instead of
            // in every compute wave
            float* cpl = reinterpret_cast<float*>(lds + L::CPL) + slot * 512;
            *reinterpret_cast<floatx4*>(cpl + 256 + 4 * lane) = mt(a10, TT1);
            if constexpr (NBW > 0) flag_set(flags + 1, x + 1);
        };
        // Phase B, part 2: the chunk's 1/||k|| and 1/||q|| (for the recurrence)
        // and Aqk's block 0
        auto phase_p2 = [&](int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4;
            const int slot = opaque_uniform(x & 1);
            unsigned char* rec = lds + L::REC + opaque_uniform(x % 3) * R::BYTES;
            // 1/||k|| (lanes 0..31) and 1/||q|| (lanes 32..63) of the chunk's
            // tokens; 0 for padding
            float* invn = reinterpret_cast<float*>(lds + L::INVN) + opaque_uniform(x % 3) * 64;
            {
                const float* nr = reinterpret_cast<const float*>(lds + L::NRM) + slot * NPW * 64;
                float v = nr[lane];
#pragma unroll
                for (int pp = 1; pp < NPW; ++pp) v += nr[pp * 64 + lane];
                const int nvalid = nvalid_of(x);
                invn[lane] = (lane & 31) < nvalid ? rsq_hw(v + NORM_EPS) : 0.f;
            }
            const floatx4 aq = build_aq(slot, 0, tile(slot, 2, lane), m, g);
            const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<bf16xEL*>(rec + R::AQK + lane * (2 * EL)) = pack_tok(aq, zero);
            if constexpr (NBW > 0) {
                // Tb10 = -(T11 A10) Tb00 once, into the record (the compute
                // waves, which set the pace here, read it), after parts 0 and
                // 1 have left their fp32 tiles
                flag_wait(flags, x + 1);
                flag_wait(flags + 1, x + 1);
                const float* cpl = reinterpret_cast<const float*>(lds + L::CPL) + slot * 512;
                floatx4 tb00d;  // Tb00[4g + i][m]
#pragma unroll
                for (int i = 0; i < 4; ++i) tb00d[i] = cpl[16 * (4 * g + i) + m];
                const floatx4 ta = *reinterpret_cast<const floatx4*>(cpl + 256 + 4 * lane);
                const floatx4 c = mt(tb00d, ta);
                bf16x4 t10;
#pragma unroll
                for (int i = 0; i < 4; ++i) t10[i] = (bf16)(-c[i]);
                *reinterpret_cast<bf16x4*>(rec + R::TB + (64 + lane) * (2 * EL)) = t10;
            }
        };
        // Phase B, part 3: Aqk's block 1 and the decay bound of warm-up chunks
        auto phase_p3 = [&](int x) __attribute__((always_inline)) {
            const int lane = opaque_lane(), m = lane & 15, g = lane >> 4;
            const int slot = opaque_uniform(x & 1);
            unsigned char* rec = lds + L::REC + opaque_uniform(x % 3) * R::BYTES;
            const float* bs = reinterpret_cast<const float*>(lds + L::BETA) + slot * 32;
            const floatx4 aq = build_aq(slot, 1, tile(slot, 3, lane), m, g);
            // Aqk block 1 = [Aqk10 | Aqk11] (Aqk10: all keys before the query)
            *reinterpret_cast<bf16xEL*>(rec + R::AQK + (64 + lane) * (2 * EL)) =
                pack_tok(tile(slot, 5, lane), aq);
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
            const unsigned char* buf = lds + L::REC + opaque_uniform(x % 3) * R::BYTES;
            const int nvalid = nvalid_of(x);
            const bool outs = x >= out_from;
            const bool want_o = outs && (!STORE || a.o != nullptr);
            // the entering state, rounded to bf16 as for the products below,
            // into chunk_state [slots, H, K, V], first (only the fp32 state is
            // live yet).  A lane holds columns 2 lr, 2 lr + 1 of its channels;
            // the lanes of a pair swap one word per two channels, so that each
            // writes four adjacent columns of one channel: 8-byte stores, half
            // as many as with the lane's own pairs
            if constexpr (STORE && CT == 2) {
                if (outs) {
                    const int64_t sslot = (int64_t)n * ((a.T + C - 1) / C) + x0 + x;
                    char* sbase = reinterpret_cast<char*>(a.chunk_state + (sslot * a.H + h) * K * V);
                    const bool odd = lr & 1;
                    const uint32_t cpair = (uint32_t)col_of(0, lr & ~1);
                    auto pk = [](float lo, float hi) __attribute__((always_inline)) {
                        return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)lo) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)hi) << 16);
                    };
#pragma unroll
                    for (int t = 0; t < KT; ++t)
#pragma unroll
                        for (int i = 0; i < 4; i += 2) {
                            const uint32_t w0 = pk(S[0][t][i], S[1][t][i]);
                            const uint32_t w1 = pk(S[0][t][i + 1], S[1][t][i + 1]);
                            // quad_perm [1, 0, 3, 2]: the pair partner's word
                            const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(
                                0, (int)(odd ? w0 : w1), 0xB1, 0xf, 0xf, false);
                            const uint32_t ch = (uint32_t)tile_channel(t, 4 * lg + i + (odd ? 1 : 0));
                            const uint2 val = odd ? uint2{recv, w1} : uint2{w0, recv};
                            *reinterpret_cast<uint2*>(sbase + (ch * V + cpair) * 2u) = val;
                        }
                }
            }
            // 1/||k|| of the lane's tokens 16 bb + 4 lg + i (the record holds the
            // raw keys and queries; phase B wrote these for the chunk)
            const float* invn = reinterpret_cast<const float*>(lds + L::INVN) + opaque_uniform(x % 3) * 64;
            const floatx4 ikt[2] = {*reinterpret_cast<const floatx4*>(invn + 4 * lg),
                                    *reinterpret_cast<const floatx4*>(invn + 16 + 4 * lg)};
            // (first: its fp32 MFMA chain depends on phase B's tiles only)
            // Tb's block 1 = [Tb10 | Tb11]: Tb10 = -(T11 A10) Tb00 from phase
            // B's fp32 tiles (the same in every compute wave), Tb11 from the record
            bf16xEL tb1 = *reinterpret_cast<const bf16xEL*>(buf + R::TB + (64 + lane) * (2 * EL));
            if constexpr (NBW == 0) {
                const float* cpl = reinterpret_cast<const float*>(lds + L::CPL) + opaque_uniform(x & 1) * 512;
                floatx4 tb00d;  // Tb00[4g + i][m]
#pragma unroll
                for (int i = 0; i < 4; ++i) tb00d[i] = cpl[16 * (4 * lg + i) + lr];
                const floatx4 ta = *reinterpret_cast<const floatx4*>(cpl + 256 + 4 * lane);
                // M(Tb00, (T11 A10)^T) = (T11 A10 Tb00)^T: element i is [m][4g + i]
                const floatx4 c = mt(tb00d, ta);
#pragma unroll
                for (int i = 0; i < 4; ++i) tb1[i] = (bf16)(-c[i]);
            }
            // Y_b = V_b - KG_b S and O^T = S^T QG^T
            const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
            floatx4 Y[CT][2], OT[CT][2];
            if constexpr (NBW > 0) {
                // with phase-B waves (168 registers a wave): one 32-channel slice
                // of S at a time, its bf16 operand formed just before its products
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb) Y[ct][bb] = OT[ct][bb] = zero;
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    bf16x8 sb[CT];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            sb[ct][e] = (bf16)S[ct][2 * j][e];
                            sb[ct][4 + e] = (bf16)S[ct][2 * j + 1][e];
                        }
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb) {
                        const bf16x8 kgo = *reinterpret_cast<const bf16x8*>(
                            buf + R::NKG + ((bb * KS + j) * 64 + lane) * 16);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) Y[ct][bb] = mfma32(kgo, sb[ct], Y[ct][bb]);
                    }
                    if (want_o) {
#pragma unroll
                        for (int ob = 0; ob < 2; ++ob) {
                            const bf16x8 qg = *reinterpret_cast<const bf16x8*>(
                                buf + R::QG + ((ob * KS + j) * 64 + lane) * 16);
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct) OT[ct][ob] = mfma32(sb[ct], qg, OT[ct][ob]);
                        }
                    }
                }
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t w = vin.w[bb][i];
                        Y[0][bb][i] = fmaf(-ikt[bb][i], Y[0][bb][i], bf_lo(w));
                        if constexpr (CT == 2) Y[1][bb][i] = fmaf(-ikt[bb][i], Y[1][bb][i], bf_hi(w));
                    }
            } else {
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
                // Y_b = V_b - KG_b S: the product with the raw keys (the record's
                // nKG slot holds +KG in this pass), then per token V - (1/||k||) K G S
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb) Y[ct][bb] = zero;
#pragma unroll
                for (int j = 0; j < KS; ++j)
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb) {
                        const bf16x8 kgo = *reinterpret_cast<const bf16x8*>(
                            buf + R::NKG + ((bb * KS + j) * 64 + lane) * 16);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) Y[ct][bb] = mfma32(kgo, sb[ct][j], Y[ct][bb]);
                    }
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t w = vin.w[bb][i];
                        Y[0][bb][i] = fmaf(-ikt[bb][i], Y[0][bb][i], bf_lo(w));
                        if constexpr (CT == 2) Y[1][bb][i] = fmaf(-ikt[bb][i], Y[1][bb][i], bf_hi(w));
                    }
                // O^T = S^T QG^T (+ U'^T Aqk^T below), raw queries: scaled by
                // 1/||q|| at the store
                if (want_o) {
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
            }
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
            // U' = Tb Y over the chunk's tokens
            bf16xEL yc[CT], uc[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    yc[ct][i] = (bf16)Y[ct][0][i];
                    yc[ct][4 + i] = (bf16)Y[ct][1][i];
                }
            if constexpr (STORE) {
                // V - KG S into chunk_u [slots, H, V, C]: token 16 bb + 4 lg + i
                // of column col_of(ct, lr) at position 8 lg + 4 bb + i (the
                // k-slot order of the 32-token operands), 16 bytes a tile
                if (outs) {
                    const int64_t sslot = (int64_t)n * ((a.T + C - 1) / C) + x0 + x;
                    char* ubase = reinterpret_cast<char*>(a.chunk_u + (sslot * a.H + h) * V * C);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        *reinterpret_cast<bf16xEL*>(
                            ubase + ((uint32_t)col_of(ct, lr) * C + 8u * lg) * 2u) = yc[ct];
                }
            }
            floatx4 U[CT][2];
            {
                const bf16xEL tb0 = *reinterpret_cast<const bf16xEL*>(buf + R::TB + lane * (2 * EL));
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    U[ct][0] = mfma_tok(tb0, yc[ct], zero);
                    U[ct][1] = mfma_tok(tb1, yc[ct], zero);
                }
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // (1/||k_t||) U'_t: the record's Kd and Aqk hold the raw keys
                    uc[ct][i] = (bf16)(U[ct][0][i] * ikt[0][i]);
                    uc[ct][4 + i] = (bf16)(U[ct][1][i] * ikt[1][i]);
                }
            // S = Diag(Gam_C) S + KdT U'.  Unit t * 64 + lane of KdT sits at
            // st_unit(t * 64 + lane) = t * 64 + (lane ^ g): one lane offset,
            // the tile's as an instruction immediate
            const unsigned char* kdtl = buf + R::KDT + (lane ^ lg) * 16;
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const bf16xEL kdt = *reinterpret_cast<const bf16xEL*>(kdtl + t * 1024);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) S[ct][t] = mfma_tok(kdt, uc[ct], S[ct][t]);
            }
            if (!want_o) return;
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                const bf16xEL aqk =
                    *reinterpret_cast<const bf16xEL*>(buf + R::AQK + (ob * 64 + lane) * (2 * EL));
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) OT[ct][ob] = mfma_tok(uc[ct], aqk, OT[ct][ob]);
            }
            // OT[ct][ob][i] = O[token 16 ob + lr][column of tile ct, tile row 4 lg + i]
            // (a wave-uniform base and 32-bit lane offsets, as for the loads)
            char* obase = reinterpret_cast<char*>(a.o + row0 * V) + chunk_off(x, 2u * V);
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                if (16 * ob + lr >= nvalid) continue;
                uint16_t* op = reinterpret_cast<uint16_t*>(
                    obase + (uint32_t)(16 * ob + lr) * (uint32_t)(a.H * V) * 2u);
                const float so = a.scale * invn[32 + 16 * ob + lr];  // scale / ||q||
                if constexpr (CT == 2) {
                    // tile ct row 4 lg + i is column wcol + 2 (4 lg + i) + ct: the
                    // lane's 8 values are columns wcol + 8 lg .. + 7
                    bf16x8 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ov[2 * i] = (bf16)(so * OT[0][ob][i]);
                        ov[2 * i + 1] = (bf16)(so * OT[1][ob][i]);
                    }
                    *reinterpret_cast<bf16x8*>(op + wcol + 8 * lg) = ov;
                } else {
                    bf16x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov[i] = (bf16)(so * OT[0][ob][i]);
                    *reinterpret_cast<bf16x4*>(op + wcol + 4 * lg) = ov;
                }
            }
        };

    // phase B of chunk x, part (w - x) mod 4 on wave w of its role: parts 0
    // and 1 (the substitutions) on SIMDs two apart
    auto phase_b = [&](int w, int x) __attribute__((always_inline)) {
        const int part = (w - x) & (NCW - 1);
        if (part == 0) phase_p0(x);
        else if (part == 2) phase_p1(x);
        else if (part == 1) phase_p2(x);
        else phase_p3(x);
    };

    // ------------------------------------------------------- the iterations
    // Iteration it (from -2 to n_it - 1): compute chunk it, phase B chunk it+1
    // and the loads of v for chunk it+2; the loads of q, k, g and beta for
    // chunk it+3 (chunk 0 before the loop) and phase A of chunk it+2.
    // Each role runs its own copy of the loop (the same iterations and
    // barriers), unrolled by three so that every register ring slot is a
    // constant; both leave it after iteration n_it - 1.
    if (is_cw) {
        for (int attempt = 0; attempt < N_ATTEMPTS; ++attempt) {
            begin_attempt(attempt);
            load_state(exact);
            if (tid == 0) {
                misc[0] = 0.f;  // sum of the warm-up chunks' bounds
                flags[0] = flags[1] = 0;
            }
            if (n_it <= 0) break;
            const int n_iter = (n_it + 2 + 2) / 3 * 3;
            VIn vin[3];
            bool restart = false, done = false;
            for (int k3 = 0; k3 < n_iter && !restart && !done; k3 += 3) {
                static_for<0, 3>([&](auto u) __attribute__((always_inline)) {
                    if (restart || done) return;
                    const int it = k3 + u - 2;
                    done = it >= n_it;  // the unrolled tail: no work, no barrier
                    if (done) return;
                    if (failed_bound(it)) {
                        restart = true;
                        return;
                    }
                    // ring slot of chunk y: y mod 3
                    constexpr int sv = u, sc = (u + 1) % 3;
                    // unconditional (a valid chunk re-read at the ends): a load
                    // issued on some paths only makes the compiler's in-order
                    // wait counts cover the loads just issued as well
                    load_v(vin[sv], min(it + 2, n_it - 1));
                    // (the last chunk's phase B runs on the prep waves, idle by then)
                    if (NBW == 0 && it + 1 >= 0 && it + 1 < n_it - 1) phase_b(wave, it + 1);
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
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float* rp = fp + tile_channel(t, 4 * lg + i) * V + col_of(0, lr);
                    if constexpr (CT == 2) *reinterpret_cast<float2*>(rp) = float2{S[0][t][i], S[1][t][i]};
                    else *rp = S[0][t][i];
                }
        }
    } else if (is_bw) {
        // phase-B waves (scalar gate): the same iterations and barriers
        for (int attempt = 0; attempt < N_ATTEMPTS; ++attempt) {
            begin_attempt(attempt);
            if (n_it <= 0) break;
            const int n_iter = (n_it + 2 + 2) / 3 * 3;
            bool restart = false, done = false;
            for (int k3 = 0; k3 < n_iter && !restart && !done; k3 += 3) {
                static_for<0, 3>([&](auto u) __attribute__((always_inline)) {
                    if (restart || done) return;
                    const int it = k3 + u - 2;
                    done = it >= n_it;
                    if (done) return;
                    if (failed_bound(it)) {
                        restart = true;
                        return;
                    }
                    if (it + 1 >= 0 && it + 1 < n_it) phase_b(wave - NCW, it + 1);
                    __syncthreads();
                });
            }
            if (!restart) break;
            __syncthreads();
        }
    } else {
        for (int attempt = 0; attempt < N_ATTEMPTS; ++attempt) {
            begin_attempt(attempt);
            if (n_it <= 0) break;
            const int n_iter = (n_it + 2 + 2) / 3 * 3;
            // nothing in flight on entry (a restarted attempt leaves loads of
            // the abandoned one): the loop's wait counts hold on every path
            __builtin_amdgcn_s_waitcnt(VMCNT_0);
            PIn pin[3];
            load_in(pin[0], 0);
            bool restart = false, done = false;
            for (int k3 = 0; k3 < n_iter && !restart && !done; k3 += 3) {
                static_for<0, 3>([&](auto u) __attribute__((always_inline)) {
                    if (restart || done) return;
                    const int it = k3 + u - 2;
                    done = it >= n_it;  // as in the compute waves' loop
                    if (done) return;
                    if (failed_bound(it)) {
                        restart = true;
                        return;
                    }
                    constexpr int sa = u, sl = (u + 1) % 3;  // ring slot of chunk y: y mod 3
                    // one chunk ahead: the loads have the rest of this phase A
                    // and the barrier to land (two ahead measured no faster in
                    // the steady state, and the first iteration then waited on
                    // a burst of both chunks from every workgroup at once);
                    // unconditional (see load_v)
                    auto loads = [&]() __attribute__((always_inline)) {
                        load_in(pin[sl], min(it + 3, n_it - 1));
                    };
                    if (it + 2 < n_it) {
                        phase_a(pin[sa], it + 2, loads);
                    } else {
                        loads();
                        touch(pin[sa]);
                        if (NBW == 0 && it + 1 == n_it - 1) {
                            // all four parts over the K/32 prep waves
#pragma unroll
                            for (int w = 0; w < NCW; w += NPW) phase_b(p + w, it + 1);
                        }
                    }
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
    using Lay = FusedLayout<K, V, GDN>;
    const dim3 grid((unsigned)n_groups), block(Lay::NT);
    if constexpr (!GDN && Lay::CT == 2) {
        if (a.chunk_state) {
            hipLaunchKernelGGL((kda_fused_kernel<K, V, false, true>), grid, block, 0, stream, a);
            return;
        }
    }
    if (ev)
        hipExtLaunchKernelGGL((kda_fused_kernel<K, V, GDN, false>), grid, block, 0, stream,
                              ev->start, ev->stop, 0, a);
    else
        hipLaunchKernelGGL((kda_fused_kernel<K, V, GDN, false>), grid, block, 0, stream, a);
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
