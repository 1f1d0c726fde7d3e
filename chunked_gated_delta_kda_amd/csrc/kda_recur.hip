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
// the record and of the chunk's V tile DEPTH+2 chunks ahead into registers;
// two chunks ahead the slices are written to one of three LDS buffers; one
// chunk ahead each wave reads its MFMA operands from LDS into registers, so
// the chunk being computed reads only its decay vector.  One barrier per
// chunk.
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
    static_assert(DEPTH % 2 == 0 && DEPTH >= 2, "the operand double buffer needs an even depth");
    using R = Rec<K>;
    using L = StageLayout<K, NW>;
    constexpr int KS = K / 32, KT = K / 16;
    __shared__ __attribute__((aligned(16))) unsigned char stage[3][L::PADDED];

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

    // state tiles: S[t][i] = S[rho(t, 4 lg + i)][cb + cw + lr] (channel order of kda_common.h)
    floatx4 S[KT];
    const int64_t st = ((int64_t)n * a.H + h) * K * a.V + cb + cw + lr;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[t][i] = a.initial_state
                          ? a.initial_state[st + (int64_t)tile_channel(t, 4 * lg + i) * a.V]
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
    // Per-lane parts of the addresses are fixed; only the chunk's base moves.
    int64_t lane_off[L::PPL];
    int lane_tok[L::PPL];
    bool lane_rec[L::PPL];
#pragma unroll
    for (int j = 0; j < L::PPL; ++j) {
        const int p = min(j * L::THREADS + tid, L::PIECES - 1);
        lane_rec[j] = p < L::REC_PIECES;
        const int q = max(p - L::REC_PIECES, 0);
        lane_tok[j] = q / L::VPR;
        lane_off[j] = lane_rec[j] ? (int64_t)p * 16
                                  : ((int64_t)lane_tok[j] * vstride + (q % L::VPR) * 8) * 2;
    }
    auto issue = [&](u32x4 (&dst)[L::PPL], int c) {
        c = min(c, nch - 1);
        const unsigned char* rec = rec_h + (int64_t)(s0 + c) * rec_stride;
        const int64_t start = t0 + (int64_t)C * c;
        const int nvalid = (int)min((int64_t)C, t1 - start);
        const unsigned char* vb = reinterpret_cast<const unsigned char*>(vcol + start * vstride);
#pragma unroll
        for (int j = 0; j < L::PPL; ++j) {
            // a V slice of a token past the end re-reads the chunk's first token
            const int64_t off = (lane_rec[j] || lane_tok[j] < nvalid)
                                    ? lane_off[j]
                                    : lane_off[j] - (int64_t)lane_tok[j] * vstride * 2;
            dst[j] = *reinterpret_cast<const u32x4*>((lane_rec[j] ? rec : vb) + off);
        }
    };
    // Slices past the end land in the buffer's padding.
    auto commit = [&](const u32x4 (&src)[L::PPL], unsigned char* buf) {
#pragma unroll
        for (int j = 0; j < L::PPL; ++j)
            *reinterpret_cast<u32x4*>(buf + (j * L::THREADS + tid) * 16) = src[j];
    };

    // nKG, the first operand on the state's critical path, is read from the
    // chunk's LDS buffer one chunk ahead of use; everything else is read from
    // the chunk's own buffer while its products run.
    struct Frags {
        bf16x8 nkg[NB][KS];
    };
    auto read_frags = [&](Frags& f, const unsigned char* buf) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < KS; ++j)
                f.nkg[b][j] = *reinterpret_cast<const bf16x8*>(
                    buf + R::NKG + ((b * KS + j) * 64 + lane) * 16);
    };

    // One chunk: nKG from registers, the rest from the chunk's buffer.
    auto compute = [&](const Frags& f, const unsigned char* buf, int c) {
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
        // -KG_b S for each 16-token block b
        floatx4 Y[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            Y[b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) Y[b] = mfma32(f.nkg[b][j], sb[j], Y[b]);
        }
        // O_ob^T = S^T QG_ob^T for each 16-token output block ob
        floatx4 OT[NB];
#pragma unroll
        for (int ob = 0; ob < NB; ++ob) {
            OT[ob] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                const bf16x8 qg = *reinterpret_cast<const bf16x8*>(
                    buf + R::QG + ((ob * KS + j) * 64 + lane) * 16);
                OT[ob] = mfma32(sb[j], qg, OT[ob]);
            }
        }
        // decay the state; the rank-C update accumulates onto it
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const floatx4 gc =
                *reinterpret_cast<const floatx4*>(buf + R::GAMC + (16 * t + 4 * lg) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t][i] *= gc[i];
        }
        // Y_b = V_b - KG_b S (padding tokens read 0)
        const uint16_t* vt = reinterpret_cast<const uint16_t*>(buf + L::V_OFF);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * b + 4 * lg + i;
                const float v = bf2f(vt[tok * L::VCOLS + cw + lr]);
                Y[b][i] += tok < nvalid ? v : 0.f;
            }
        // U' = Tb Y over the chunk's tokens, one 16-token row block at a time
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        bf16xEL yc, uc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            yc[i] = (bf16)Y[0][i];
            if constexpr (NB == 2) yc[4 + i] = (bf16)Y[NB - 1][i];
        }
        floatx4 U[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const bf16xEL tb =
                *reinterpret_cast<const bf16xEL*>(buf + R::TB + (b * 64 + lane) * (2 * EL));
            U[b] = mfma_tok(tb, yc, zero);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uc[i] = (bf16)U[0][i];
            if constexpr (NB == 2) uc[4 + i] = (bf16)U[NB - 1][i];
        }
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const bf16xEL kdt =
                *reinterpret_cast<const bf16xEL*>(buf + R::KDT + (t * 64 + lane) * (2 * EL));
            S[t] = mfma_tok(kdt, uc, S[t]);
        }
        // + U'^T Aqk^T.  With one block the 16x16x16 product is accumulated apart
        // and added on the VALU: a 16x16x16 MFMA must not take the result of a
        // 16x16x32 MFMA as its accumulator input (that dependent pair gave wrong
        // sums on gfx950).  With two blocks both products are 16x16x32.
#pragma unroll
        for (int ob = 0; ob < NB; ++ob) {
            const bf16xEL aqk =
                *reinterpret_cast<const bf16xEL*>(buf + R::AQK + (ob * 64 + lane) * (2 * EL));
            if constexpr (NB == 1) {
                const floatx4 OI = mfma_tok(uc, aqk, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) OT[ob][i] += OI[i];
            } else {
                OT[ob] = mfma_tok(uc, aqk, OT[ob]);
            }
            // OT[ob][i] = O[token 16 ob + lr][column cb + cw + 4 lg + i]
            if (16 * ob + lr < nvalid) {
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = (bf16)(a.scale * OT[ob][i]);
                *reinterpret_cast<bf16x4*>(a.o + (start + 16 * ob + lr) * vstride +
                                           (int64_t)h * a.V + cb + cw + 4 * lg) = ov;
            }
        }
    };

    if (nch > 0) {
        // Pipeline, iteration c: chunk c + 2 + DEPTH loads into registers,
        // chunk c + 2 is written to LDS buffer (c + 2) % 3, chunk c + 1's nKG is
        // read from buffer (c + 1) % 3 into registers, and chunk c computes
        // (reading its other operands from buffer c % 3).  One barrier.
        Frags fr[2];
        static_for<0, DEPTH>([&](auto d) { issue(ring[d], d); });
        commit(ring[0], stage[0]);
        commit(ring[1 % DEPTH], stage[1]);
        __syncthreads();
        issue(ring[0], DEPTH);
        issue(ring[1 % DEPTH], DEPTH + 1);
        read_frags(fr[0], stage[0]);
        int sc = 0;  // buffer of chunk c: c % 3
        for (int base = 0; base < nch; base += DEPTH) {
            static_for<0, DEPTH>([&](auto u) {
                constexpr int nx2 = (u + 2) % DEPTH;  // ring slot of chunk c + 2
                constexpr int cur = u & 1;            // DEPTH is even
                const int c = base + u;
                const int s1b = sc == 2 ? 0 : sc + 1, s2b = sc == 0 ? 2 : sc - 1;
                commit(ring[nx2], stage[s2b]);  // chunk c + 2
                issue(ring[nx2], c + 2 + DEPTH);
                read_frags(fr[cur ^ 1], stage[s1b]);          // chunk c + 1
                if (c < nch) compute(fr[cur], stage[sc], c);  // uniform over the workgroup
                __syncthreads();
                sc = s1b;
            });
        }
    }

    if (a.final_state) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.final_state[st + (int64_t)tile_channel(t, 4 * lg + i) * a.V] = S[t][i];
    }
}

// Waves per workgroup (16 value columns each) and prefetch depth in chunks.
#ifndef KDA_RECUR_WAVES
#define KDA_RECUR_WAVES 4
#endif
#ifndef KDA_RECUR_DEPTH
#define KDA_RECUR_DEPTH 2
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
