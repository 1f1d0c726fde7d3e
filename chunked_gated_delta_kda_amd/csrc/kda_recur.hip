// kda_recur.hip -- head-parallel half of the chunked forward pass (gfx950).
//
// One workgroup per (sequence, head, block of 16 * NW value columns); each
// wave owns 16 value columns of the [K, V] state, kept in fp32 MFMA
// accumulators for the whole sequence.  Columns of S evolve independently
// (the recurrence only mixes rows), so splitting V is exact.
//
// Per chunk (records from kda_prep, notation of kda_common.h), with S the
// state entering the chunk:
//   Y   = V - KG S                    16x16x32 MFMA, K/32 steps
//   U'  = Tb Y                        the chunk's true per-token updates
//   O^T = S^T QG^T + U'^T Aqk^T       output for the 16 tokens, scaled
//   S   = Diag(Gam_C) S + KdT U'      16x16x16 MFMA, K/16 tiles
// This is the chunkwise form of S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1}
// + b_t k_t v_t^T, o_t = scale S_t^T q_t: unrolling the recurrence over a
// chunk gives (I + A) U' = diag(b)(V - (K^*Gam) S).  The FlashKDA summary
// (discuss.pytorch.kr, section "커널 퓨전(Kernel Fusion) 전략의 분리") assigns this
// recurrence and the output projection to its second, head-parallel kernel.
//
// The state tiles' D layout is, element for element, the operand layout the
// next chunk needs (k index order of kda_common.h), so the loop has no
// transposes; the only conversions are fp32 -> bf16 of the operand copies.
//
// Memory pipeline: the loop is a strict chain (chunk i+1 needs the state
// after chunk i), so the HBM latency of the per-chunk inputs must be hidden
// by loading far ahead.  Every lane of the workgroup loads a 16-byte slice of
// the record and of the chunk's V tile DEPTH chunks ahead into registers; one
// chunk ahead the slices are written to an LDS double buffer from which the
// waves read their MFMA fragments.  One barrier per chunk.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

template <int K, int NW>
struct StageLayout {
    using R = Rec<K>;
    static constexpr int VCOLS = 16 * NW;               // value columns per workgroup
    static constexpr int VBYTES = C * VCOLS * 2;        // V tile, bf16 [C][VCOLS]
    static constexpr int V_OFF = R::BYTES;              // V tile after the record
    static constexpr int BYTES = R::BYTES + VBYTES;
    static constexpr int PIECES = BYTES / 16;           // 16-byte slices per chunk
    static constexpr int REC_PIECES = R::BYTES / 16;
    static constexpr int THREADS = 64 * NW;
    static constexpr int PPL = (PIECES + THREADS - 1) / THREADS;  // slices per lane
    static constexpr int VPR = VCOLS * 2 / 16;          // 16-byte slices per V token row
    static constexpr int PADDED = PPL * THREADS * 16;   // LDS bytes per buffer
};

template <int K, int NW, int DEPTH>
__global__ __launch_bounds__(64 * NW) void kda_recur_kernel(RecurArgs a) {
    using R = Rec<K>;
    using L = StageLayout<K, NW>;
    constexpr int KS = K / 32, KT = K / 16;
    __shared__ __attribute__((aligned(16))) unsigned char stage[2][L::PADDED];

    // XCD-aware placement: workgroups are dealt to the 8 XCDs round robin, so
    // blocks b and b + 8 share an XCD (and its L2).  The VS column blocks of
    // one (sequence, head) read the same records; give them indices that
    // differ by multiples of 8.
    const int VS = a.V / L::VCOLS;
    const int b = blockIdx.x;
    const int pair = (b / (8 * VS)) * 8 + (b & 7);
    const int vs = (b >> 3) % VS;
    if (pair >= a.n_seqs * a.H) return;  // grid padded to a multiple of 8 * VS
    const int h = pair % a.H, n = pair / a.H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int cw = wave * 16;            // this wave's first column within the block
    const int cb = vs * L::VCOLS;        // the block's first value column

    // state tiles: S[t][i] = S[16 t + 4 lg + i][cb + cw + lr]
    floatx4 S[KT];
    const int64_t st = ((int64_t)n * a.H + h) * K * a.V + cb + cw + lr;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[t][i] = a.initial_state ? a.initial_state[st + (int64_t)(16 * t + 4 * lg + i) * a.V]
                                      : 0.f;

    int64_t t0, t1;
    int s0, s1;
    seq_span(a, n, t0, t1, s0, s1);
    const int nch = s1 - s0;
    const int64_t vstride = (int64_t)a.H * a.V;  // elements between consecutive tokens
    const unsigned char* rec_h = a.rec + (int64_t)h * R::BYTES;
    const int64_t rec_stride = (int64_t)a.H * R::BYTES;
    const uint16_t* vcol = a.v + (int64_t)h * a.V + cb;

    // Register ring: slice j of chunk c lives in ring[c % DEPTH][j].
    u32x4 ring[DEPTH][L::PPL];

    // Loads this lane's slices of chunk c (clamped to the last chunk, so the
    // pipeline can run past the end with harmless re-reads).  Every lane issues
    // exactly PPL loads per chunk with no branch: slice indices past the end
    // re-read the last slice, and V slices past the chunk's last token re-read
    // its first token.  Straight-line loads let the compiler count them and
    // wait for exactly the oldest chunk instead of draining the queue.
    auto issue = [&](u32x4 (&dst)[L::PPL], int c) {
        c = min(c, nch - 1);
        const unsigned char* rec = rec_h + (int64_t)(s0 + c) * rec_stride;
        const int64_t start = t0 + (int64_t)C * c;
        const int nvalid = (int)min((int64_t)C, t1 - start);
#pragma unroll
        for (int j = 0; j < L::PPL; ++j) {
            const int p = min(j * L::THREADS + tid, L::PIECES - 1);
            const int q = max(p - L::REC_PIECES, 0);
            int tok = q / L::VPR;
            tok = tok < nvalid ? tok : 0;
            const unsigned char* vaddr = reinterpret_cast<const unsigned char*>(
                vcol + (start + tok) * vstride + (q % L::VPR) * 8);
            const unsigned char* addr = p < L::REC_PIECES ? rec + p * 16 : vaddr;
            dst[j] = *reinterpret_cast<const u32x4*>(addr);
        }
    };
    // Slices past the end land in the buffer's padding.
    auto commit = [&](const u32x4 (&src)[L::PPL], unsigned char* buf) {
#pragma unroll
        for (int j = 0; j < L::PPL; ++j)
            *reinterpret_cast<u32x4*>(buf + (j * L::THREADS + tid) * 16) = src[j];
    };

    // One chunk, every operand read from the LDS buffer.
    auto compute = [&](const unsigned char* buf, int c) {
        const int64_t start = t0 + (int64_t)C * c;
        const int nvalid = (int)min((int64_t)C, t1 - start);
        // bf16 operand copy of the state: k-step j pairs tiles 2j and 2j+1
        bf16x8 sb[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sb[j][e] = (bf16)S[2 * j][e];
                sb[j][4 + e] = (bf16)S[2 * j + 1][e];
            }
        // decay the state now; the rank-C update accumulates onto it below
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const floatx4 gc =
                *reinterpret_cast<const floatx4*>(buf + R::GAMC + (16 * t + 4 * lg) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t][i] *= gc[i];
        }
        floatx4 Y;
        const uint16_t* vt = reinterpret_cast<const uint16_t*>(buf + L::V_OFF);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 4 * lg + i;
            Y[i] = tok < nvalid ? bf2f(vt[tok * L::VCOLS + cw + lr]) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const bf16x8 nkg =
                *reinterpret_cast<const bf16x8*>(buf + R::NKG + (j * 64 + lane) * 16);
            Y = mfma32(nkg, sb[j], Y);  // V - KG S
        }
        floatx4 OT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const bf16x8 qg = *reinterpret_cast<const bf16x8*>(buf + R::QG + (j * 64 + lane) * 16);
            OT = mfma32(sb[j], qg, OT);  // S^T QG^T
        }
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        const bf16x4 tb = *reinterpret_cast<const bf16x4*>(buf + R::TB + lane * 8);
        const bf16x4 ub = to_bf16x4(mfma16(tb, to_bf16x4(Y), zero));  // U'
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const bf16x4 kdt =
                *reinterpret_cast<const bf16x4*>(buf + R::KDT + (t * 64 + lane) * 8);
            S[t] = mfma16(kdt, ub, S[t]);
        }
        // + U'^T Aqk^T, accumulated apart and added on the VALU: a 16x16x16 MFMA
        // must not take the result of a 16x16x32 MFMA as its accumulator input
        // (that dependent pair gave wrong sums on gfx950)
        const bf16x4 aqk = *reinterpret_cast<const bf16x4*>(buf + R::AQK + lane * 8);
        const floatx4 OI = mfma16(ub, aqk, zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) OT[i] += OI[i];
        // OT[i] = O[token lr][column cb + cw + 4 lg + i]
        if (lr < nvalid) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (bf16)(a.scale * OT[i]);
            *reinterpret_cast<bf16x4*>(a.o + (start + lr) * vstride + (int64_t)h * a.V + cb + cw +
                                       4 * lg) = ov;
        }
    };

    if (nch > 0) {
        // prologue: chunks 0 .. DEPTH-1 in flight, chunk 0 staged
        static_for<0, DEPTH>([&](auto d) { issue(ring[d], d); });
        commit(ring[0], stage[0]);
        __syncthreads();
        issue(ring[0], DEPTH);
        for (int base = 0; base < nch; base += DEPTH) {
            static_for<0, DEPTH>([&](auto u) {
                constexpr int nx = (u + 1) % DEPTH;  // ring slot of chunk c + 1
                const int c = base + u;
                commit(ring[nx], stage[(c + 1) & 1]);
                issue(ring[nx], c + 1 + DEPTH);
                if (c < nch) compute(stage[c & 1], c);  // uniform over the workgroup
                __syncthreads();
            });
        }
    }

    if (a.final_state) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.final_state[st + (int64_t)(16 * t + 4 * lg + i) * a.V] = S[t][i];
    }
}

// Waves per workgroup (16 value columns each) and prefetch depth in chunks.
#ifndef KDA_RECUR_WAVES
#define KDA_RECUR_WAVES 4
#endif
#ifndef KDA_RECUR_DEPTH
#define KDA_RECUR_DEPTH 8
#endif
constexpr int RECUR_WAVES = KDA_RECUR_WAVES;
constexpr int RECUR_DEPTH = KDA_RECUR_DEPTH;

template <int K>
void launch_recur_t(const RecurArgs& a, hipStream_t stream) {
    const int vs = a.V / (16 * RECUR_WAVES);
    const int64_t pairs = (int64_t)a.n_seqs * a.H;
    const int64_t groups = (pairs + 7) / 8;  // the grid covers whole groups of 8 pairs
    hipLaunchKernelGGL((kda_recur_kernel<K, RECUR_WAVES, RECUR_DEPTH>),
                       dim3((unsigned)(groups * 8 * vs)), dim3(64 * RECUR_WAVES), 0, stream, a);
}

void launch_recur(const RecurArgs& a, int K, hipStream_t stream) {
    if (K == 128) launch_recur_t<128>(a, stream);
    else launch_recur_t<64>(a, stream);
}

}  // namespace kda
