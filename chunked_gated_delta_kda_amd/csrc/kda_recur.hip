// kda_recur.hip -- head-parallel half of the chunked forward pass (gfx950).
//
// One workgroup per (sequence, head, block of 16 * NW value columns); each
// compute wave owns 16 value columns of the [K, V] state, kept in fp32 MFMA
// accumulators for the whole sequence.  Columns of S evolve independently
// (the recurrence only mixes rows), so splitting V is exact.
//
// Per chunk (records from kda_prep, notation of kda_common.h), with S the
// state entering the chunk:
//   Y   = V - KG S                    16x16x32 MFMA, K/32 steps per block
//   U'  = Tb Y                        the chunk's true per-token updates
//   O^T = S^T QG^T + U'^T Aqk^T       output for the chunk's tokens, scaled
//   S   = Diag(Gam_C) S + KdT U'      16x16x32 MFMA over the chunk's tokens
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
// Wave roles.  The loop is a strict chain (chunk i+1 needs the state after
// chunk i), and a wave that both waits for memory and runs the chain
// serialises the two.  So the workgroup has NW compute waves and NL loader
// waves (one compute and one loader wave per SIMD at NW = NL = 4):
//   loader waves: each lane keeps 16-byte slices of the record and of the V
//     tile of DEPTH chunks in flight in registers and writes chunk c + 2 to
//     one of two LDS buffers during iteration c;
//   compute waves: during iteration c they compute chunk c and read the
//     critical-path operands of chunk c + 1 (nKG, Tb, V) into registers.
// One barrier per chunk separates the iterations.
#include <hip/hip_ext.h>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

template <int K, int NW, int CT, int NL>
struct StageLayout {
    using R = Rec<K>;
    static constexpr int VCOLS = 16 * CT * NW;          // value columns per workgroup
    static constexpr int VBYTES = C * VCOLS * 2;        // V tile, bf16 [C][VCOLS]
    static constexpr int V_OFF = R::BYTES;              // V tile after the record
    static constexpr int BYTES = R::BYTES + VBYTES;
    static constexpr int PIECES = BYTES / 16;           // 16-byte slices per chunk
    static constexpr int REC_PIECES = R::BYTES / 16;
    static constexpr int LTHREADS = 64 * NL;            // loader lanes
    static constexpr int PPL = (PIECES + LTHREADS - 1) / LTHREADS;  // slices per loader lane
    static constexpr int VPR = VCOLS * 2 / 16;          // 16-byte slices per V token row
    static constexpr int PADDED = PPL * LTHREADS * 16;  // LDS bytes per buffer
};

// OCC: workgroups per CU the register allocation must allow (launched with 1).
// MODE (RecurMode): the forward pass; the forward pass that stores, for the
// backward pass, each chunk's entering state and V - KG S (no outputs); the
// reverse pass, which walks the chunks backwards over BRec records with the
// output gradient in place of V (see kda_bwd.hip); the forward pass with its
// outputs and those stores (a forward pass whose backward pass follows).
template <int K, int NW, int CT, int NL, int DEPTH, int OCC, int MODE>
__global__ __launch_bounds__(64 * (NW + NL)) __attribute__((amdgpu_waves_per_eu(
    OCC * (NW + NL) / 4))) void kda_recur_kernel(RecurArgs a) {
    static_assert(DEPTH % 2 == 0 && DEPTH >= 2, "the loop is unrolled by DEPTH and by 2");
    constexpr bool BWD = MODE == RECUR_BWD;
    // SAVE: store each chunk's entering state and V - KG S for the backward
    // pass; OUT: compute and store the outputs
    constexpr bool SAVE = MODE == RECUR_STORE || MODE == RECUR_FWD_STORE;
    constexpr bool OUT = MODE == RECUR_FWD || MODE == RECUR_FWD_STORE;
    using R = Rec<K>;
    using BR = BRec<K>;
    using L = StageLayout<K, NW, CT, NL>;
    constexpr int KS = K / 32, KT = K / 16;
    // Two buffers: during iteration c the compute waves read chunk c + 1's
    // buffer while the loaders overwrite chunk c's, whose operands have been
    // in registers since the previous barrier.
    __shared__ __attribute__((aligned(16))) unsigned char stage[2][L::PADDED];

    // XCD-aware placement: workgroups are dealt to the 8 XCDs round robin, so
    // blocks b and b + 8 share an XCD (and its L2).  The VS column blocks of
    // one (sequence, head) read the same records; give them indices that
    // differ by multiples of 8.
    const int TC = a.trans_out ? K : 0;  // transition columns after the V value columns
    const int VS = (a.V + TC) / L::VCOLS;
    const int b = blockIdx.x;
    const int pair = (b / (8 * VS)) * 8 + (b & 7);
    const int vs = (b >> 3) % VS;
    if (pair >= a.n_seqs * a.H) return;  // grid padded to a multiple of 8 * VS
    const int h = pair % a.H, n = pair / a.H;
    const int cb = vs * L::VCOLS;  // the block's first column (value, then transition)
    // A transition block runs the recurrence on columns of the identity with
    // zero values: its final "state" is the sequence's K x K transition M, so
    // that S_end = M S_start + (the result from a zero start).
    const bool trans = cb >= a.V;

    int64_t t0, t1;
    int s0, s1;
    seq_span(a, n, t0, t1, s0, s1);
    if (a.packed) {  // a table from the workspace: keep every access inside the batch
        t0 = min(max(t0, (int64_t)0), a.tok_limit);
        t1 = min(max(t1, t0), a.tok_limit);
        s0 = min(max(s0, 0), a.slot_limit);
        s1 = min(max(s1, s0), a.slot_limit);
        s1 = (int)min((int64_t)s1, s0 + (t1 - t0 + C - 1) / C);
    }
    int nch = s1 - s0;
    if (trans) {
        // ||M||_2 <= 2^(sum of the chunk bounds): when that is negligible the
        // transition is not needed (and not computed).  Every wave reaches the
        // same decision before any barrier.
        float sum = 0.f;
        for (int c = threadIdx.x & 63; c < nch; c += 64) sum += a.bound[(int64_t)(s0 + c) * a.H + h];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
        const bool needed = !(sum < a.bound_limit);
        if (cb == a.V && threadIdx.x == 0) a.trans_flag[(int64_t)n * a.H + h] = needed ? 1 : 0;
        if (!needed) return;
    }
    // Decay window (first pass of sequence splitting, value columns): a
    // segment's end state from a zero start depends, to within
    // 2^bound_limit of the state's size, only on its trailing chunks back to
    // where their summed bounds fall below bound_limit (the product of those
    // chunks' transitions is that small), so the recurrence starts there.
    // Every wave computes the same start.
    if (a.window && !trans && nch > 0) {
        const int ln = threadIdx.x & 63;
        float acc = 0.f;
        for (int base = 0; base < nch; base += 64) {
            const int c = nch - 1 - base - ln;  // this lane's chunk, from the last back
            float x = c >= 0 ? a.bound[(int64_t)(s0 + c) * a.H + h] : 0.f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {  // suffix sums: inclusive scan over lanes
                const float y = __shfl_up(x, o, 64);
                if (ln >= o) x += y;
            }
            x += acc;
            const unsigned long long hit = __ballot(c >= 0 && x < a.bound_limit);
            if (hit) {  // uniform: keep chunks nch - w .. nch - 1
                const int w = base + __ffsll((long long)hit);
                t0 += (int64_t)C * (nch - w);
                s0 += nch - w;
                nch = w;
                break;
            }
            acc = __shfl(x, 63, 64);
        }
    }
    // Both roles run the same number of iterations (one barrier each), rounded
    // up to the unroll factor; iterations past the last chunk only synchronise.
    const int nround = (nch + DEPTH - 1) / DEPTH * DEPTH;
    const int64_t vstride = (int64_t)a.H * a.V;  // elements between consecutive tokens

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;

    if (wave >= NW) {
        // ---------------------------------------------------------- loader waves
        if (nch == 0) return;  // no barrier is reached when there is no chunk
        const int ltid = tid - 64 * NW;
        const unsigned char* rec_h = a.rec + (int64_t)h * R::BYTES;
        const int64_t rec_stride = (int64_t)a.H * R::BYTES;
        // transition blocks load a value block too (in bounds, never used)
        const uint16_t* vcol = a.v + (int64_t)h * a.V + (trans ? 0 : cb);
        // Register ring: slice j of chunk c lives in ring[c % DEPTH][j].
        u32x4 ring[DEPTH][L::PPL];
        // Every lane issues exactly PPL loads per chunk with no branch: slice
        // indices past the end re-read the last slice, and V slices past the
        // chunk's last token re-read its first token.  Straight-line loads let
        // the compiler wait for exactly the oldest chunk in flight.
        int64_t lane_off[L::PPL];
        int lane_tok[L::PPL];
        bool lane_rec[L::PPL];
#pragma unroll
        for (int j = 0; j < L::PPL; ++j) {
            const int p = min(j * L::LTHREADS + ltid, L::PIECES - 1);
            lane_rec[j] = p < L::REC_PIECES;
            const int q = max(p - L::REC_PIECES, 0);
            lane_tok[j] = q / L::VPR;
            lane_off[j] = lane_rec[j] ? (int64_t)p * 16
                                      : ((int64_t)lane_tok[j] * vstride + (q % L::VPR) * 8) * 2;
        }
        // loads chunk c (clamped to the last chunk: harmless re-reads at the end)
        auto issue = [&](u32x4 (&dst)[L::PPL], int c) {
            c = min(c, nch - 1);
            if constexpr (BWD) c = nch - 1 - c;  // the reverse pass walks backwards
            const unsigned char* rec = rec_h + (int64_t)(s0 + c) * rec_stride;
            const int64_t start = t0 + (int64_t)C * c;
            const int nvalid = (int)min((int64_t)C, t1 - start);
            const unsigned char* vb =
                reinterpret_cast<const unsigned char*>(vcol + start * vstride);
#pragma unroll
            for (int j = 0; j < L::PPL; ++j) {
                const int64_t off = (lane_rec[j] || lane_tok[j] < nvalid)
                                        ? lane_off[j]
                                        : lane_off[j] - (int64_t)lane_tok[j] * vstride * 2;
                dst[j] = *reinterpret_cast<const u32x4*>((lane_rec[j] ? rec : vb) + off);
            }
        };
        // slices past the end land in the buffer's padding
        // V rows of padding tokens (and the whole V tile of a transition block)
        // are written as zeros, so the compute waves read V without masking
        auto commit = [&](const u32x4 (&src)[L::PPL], unsigned char* buf, int c) {
            if constexpr (BWD) c = nch - 1 - min(c, nch - 1);
            const int nvalid = trans ? 0 : (int)min((int64_t)C, t1 - (t0 + (int64_t)C * c));
            const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < L::PPL; ++j)
                *reinterpret_cast<u32x4*>(buf + (j * L::LTHREADS + ltid) * 16) =
                    lane_rec[j] || lane_tok[j] < nvalid ? src[j] : zero;
        };
        static_for<0, DEPTH>([&](auto d) { issue(ring[d], d); });
        commit(ring[0], stage[0], 0);
        issue(ring[0], DEPTH);
        __syncthreads();  // chunk 0 is in buffer 0
        commit(ring[1], stage[1], 1);
        issue(ring[1], DEPTH + 1);
        __syncthreads();  // chunk 1 is in buffer 1; chunk 0's operands are in registers
        int s2b = 0;  // buffer of chunk c + 2: c % 2
        for (int base = 0; base < nround; base += DEPTH) {
            static_for<0, DEPTH>([&](auto u) {
                constexpr int nx2 = (u + 2) % DEPTH;  // ring slot of chunk c + 2
                const int c = base + u;
                // unconditional (past the end: clamped re-reads into buffers no
                // one reads), so the compiler sees a fixed order of loads and
                // waits only for the oldest chunk in flight
                commit(ring[nx2], stage[s2b], c + 2);
                issue(ring[nx2], c + 2 + DEPTH);
                __syncthreads();
                s2b ^= 1;
            });
        }
        return;
    }

    // ------------------------------------------------------------- compute waves
    const int lr = lane & 15, lg = lane >> 4;
    const int cw = wave * 16 * CT;  // this wave's first column within the block

    // state tiles: S[ct][t][i] = S[rho(t, 4 lg + i)][cb + cw + 16 ct + lr]
    // (channel order of kda_common.h)
    floatx4 S[CT][KT];
    const int64_t st = ((int64_t)n * a.H + h) * K * a.V + cb + cw + lr;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = tile_channel(t, 4 * lg + i);
                if (trans)  // identity column cb + cw + 16 ct + lr - V
                    S[ct][t][i] = row == cb + cw + 16 * ct + lr - a.V ? 1.f : 0.f;
                else
                    S[ct][t][i] =
                        a.initial_state ? a.initial_state[st + 16 * ct + (int64_t)row * a.V] : 0.f;
            }
    const bool store_o = a.o != nullptr && !trans;

    // Every operand of a chunk sits in registers when its iteration starts:
    // each fragment of chunk c + 1 is read from its LDS buffer right after
    // chunk c has used the same fragment for the last time, so the reads run
    // behind the chunk's products and the chain never waits for LDS.  Reads
    // past the last chunk are harmless (buffers are never out of bounds).
    struct Frags {
        bf16x8 nkg[NB][KS];
        bf16x8 qg[NB][KS];
        bf16xEL kdt[KT];
        bf16xEL tb[NB];
        bf16xEL aqk[NB];
        floatx4 gc[KT];
        floatx4 v[CT][NB];
    };
    auto read_nkg_v = [&](Frags& f, const unsigned char* buf) {
        const uint16_t* vt = reinterpret_cast<const uint16_t*>(buf + L::V_OFF);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
            for (int j = 0; j < KS; ++j)
                f.nkg[bb][j] = *reinterpret_cast<const bf16x8*>(
                    buf + R::NKG + ((bb * KS + j) * 64 + lane) * 16);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 16 * bb + 4 * lg + i;  // padding rows hold zeros
                    f.v[ct][bb][i] = bf2f(vt[tok * L::VCOLS + cw + 16 * ct + lr]);
                }
        }
    };
    auto read_qg = [&](Frags& f, const unsigned char* buf) {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int j = 0; j < KS; ++j)
                f.qg[bb][j] = *reinterpret_cast<const bf16x8*>(
                    buf + R::QG + ((bb * KS + j) * 64 + lane) * 16);
    };
    auto read_gc = [&](Frags& f, const unsigned char* buf) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
            f.gc[t] = *reinterpret_cast<const floatx4*>(buf + R::GAMC + (16 * t + 4 * lg) * 4);
    };
    auto read_tb = [&](Frags& f, const unsigned char* buf) {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
            f.tb[bb] =
                *reinterpret_cast<const bf16xEL*>(buf + R::TB + (bb * 64 + lane) * (2 * EL));
    };
    auto read_kdt = [&](Frags& f, const unsigned char* buf) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
            f.kdt[t] =
                *reinterpret_cast<const bf16xEL*>(buf + R::KDT + (t * 64 + lane) * (2 * EL));
    };
    auto read_aqk = [&](Frags& f, const unsigned char* buf) {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
            f.aqk[bb] =
                *reinterpret_cast<const bf16xEL*>(buf + R::AQK + (bb * 64 + lane) * (2 * EL));
    };

    // Backward-pass stores.  store_state: the bf16 state copy (k-step j of
    // column tile ct holds channels 32 j + 8 lg + e of column lr) into
    // chunk_state [slots, H, K, V].  store_tok: a [C, columns] result in D
    // layout (block bb, rows 4 lg + i) into a [slots, H, V, C] buffer with the
    // tokens in k-slot order, 8 bytes per block.
    // (single bf16 elements are taken from the packed 32-bit words with
    // integer shifts: storing vector elements of a bf16 vector directly was
    // compiled into stores of one element repeated)
    auto store_state = [&](const bf16x8 (&sb)[CT][KS], int64_t slot) {
        uint16_t* hp = a.chunk_state + (slot * a.H + h) * K * a.V + cb + cw + lr;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                const u32x4 w = __builtin_bit_cast(u32x4, sb[ct][j]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    hp[16 * ct + (int64_t)(32 * j + 8 * lg + e) * a.V] =
                        (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
    };
    auto store_tok = [&](uint16_t* base, const floatx4 (&X)[CT][NB], int64_t slot) {
        uint16_t* up = base + ((slot * a.H + h) * a.V + cb + cw + lr) * C;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
                *reinterpret_cast<bf16x4*>(up + 16 * ct * C + EL * lg + 4 * bb) =
                    to_bf16x4(X[ct][bb]);
    };

    // One chunk from registers; `next` is chunk c + 1's buffer.  Each operand
    // fragment serves the wave's CT column tiles.
    auto compute = [&](Frags& f, const unsigned char* next, int c) {
        const int64_t start = t0 + (int64_t)C * c;
        const int nvalid = (int)min((int64_t)C, t1 - start);
        // bf16 operand copy of the state: k-step j pairs tiles 2j and 2j+1
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
        if constexpr (SAVE) store_state(sb, s0 + c);
        // Y_b = V_b - KG_b S for each 16-token block b
        floatx4 Y[CT][NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) Y[ct][bb] = f.v[ct][bb];
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    Y[ct][bb] = mfma32(f.nkg[bb][j], sb[ct][j], Y[ct][bb]);
        read_nkg_v(f, next);
        if constexpr (SAVE) store_tok(a.chunk_u, Y, s0 + c);
        // O_ob^T = S^T QG_ob^T for each 16-token output block ob
        floatx4 OT[CT][NB];
        if constexpr (OUT) {
#pragma unroll
            for (int ob = 0; ob < NB; ++ob)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    OT[ct][ob] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < KS; ++j)
                        OT[ct][ob] = mfma32(sb[ct][j], f.qg[ob][j], OT[ct][ob]);
                }
            read_qg(f, next);
        }
        // decay the state; the rank-C update accumulates onto it
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[ct][t][i] *= f.gc[t][i];
        read_gc(f, next);
        // U' = Tb Y over the chunk's tokens, one 16-token row block at a time
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        bf16xEL yc[CT], uc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                yc[ct][i] = (bf16)Y[ct][0][i];
                if constexpr (NB == 2) yc[ct][4 + i] = (bf16)Y[ct][NB - 1][i];
            }
        floatx4 U[CT][NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) U[ct][bb] = mfma_tok(f.tb[bb], yc[ct], zero);
        read_tb(f, next);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uc[ct][i] = (bf16)U[ct][0][i];
                if constexpr (NB == 2) uc[ct][4 + i] = (bf16)U[ct][NB - 1][i];
            }
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) S[ct][t] = mfma_tok(f.kdt[t], uc[ct], S[ct][t]);
        read_kdt(f, next);
        if constexpr (!OUT) return;  // no outputs
        // + U'^T Aqk^T.  With one block the 16x16x16 product is accumulated apart
        // and added on the VALU: a 16x16x16 MFMA must not take the result of a
        // 16x16x32 MFMA as its accumulator input (that dependent pair gave wrong
        // sums on gfx950).  With two blocks both products are 16x16x32.
#pragma unroll
        for (int ob = 0; ob < NB; ++ob)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if constexpr (NB == 1) {
                    const floatx4 OI = mfma_tok(uc[ct], f.aqk[ob], zero);
#pragma unroll
                    for (int i = 0; i < 4; ++i) OT[ct][ob][i] += OI[i];
                } else {
                    OT[ct][ob] = mfma_tok(uc[ct], f.aqk[ob], OT[ct][ob]);
                }
            }
        read_aqk(f, next);
#pragma unroll
        for (int ob = 0; ob < NB; ++ob)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                // OT[ct][ob][i] = O[token 16 ob + lr][column cb + cw + 16 ct + 4 lg + i]
                if (store_o && 16 * ob + lr < nvalid) {
                    bf16x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov[i] = (bf16)(a.scale * OT[ct][ob][i]);
                    *reinterpret_cast<bf16x4*>(a.o + (start + 16 * ob + lr) * vstride +
                                               (int64_t)h * a.V + cb + cw + 16 * ct + 4 * lg) = ov;
                }
            }
    };

    // ---- the reverse pass (BWD): BRec operands, the output gradient in the V tile
    struct BFrags {
        bf16x8 kd[NB][KS];
        bf16xEL qgt[KT];
        bf16xEL nkgt[KT];
        bf16xEL tbt[NB];
        bf16xEL aqkt[NB];
        floatx4 gc[KT];
        floatx4 dov[CT][NB];
    };
    auto read_kd_do = [&](BFrags& f, const unsigned char* buf) {
        const uint16_t* vt = reinterpret_cast<const uint16_t*>(buf + L::V_OFF);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
            for (int j = 0; j < KS; ++j)
                f.kd[bb][j] = *reinterpret_cast<const bf16x8*>(
                    buf + BR::KD + ((bb * KS + j) * 64 + lane) * 16);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f.dov[ct][bb][i] = bf2f(vt[(16 * bb + 4 * lg + i) * L::VCOLS + cw + 16 * ct + lr]);
        }
    };
    auto read_tiles = [&](bf16xEL (&dst)[KT], const unsigned char* buf, int off) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
            dst[t] = *reinterpret_cast<const bf16xEL*>(buf + off + (t * 64 + lane) * (2 * EL));
    };
    auto read_blocks = [&](bf16xEL (&dst)[NB], const unsigned char* buf, int off) {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
            dst[bb] = *reinterpret_cast<const bf16xEL*>(buf + off + (bb * 64 + lane) * (2 * EL));
    };
    auto read_bgc = [&](BFrags& f, const unsigned char* buf) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
            f.gc[t] = *reinterpret_cast<const floatx4*>(buf + BR::GAMC + (16 * t + 4 * lg) * 4);
    };
    // One reverse step: S holds dS', the gradient of the state leaving chunk
    // cc = nch - 1 - c, and leaves with the gradient of the state entering it.
    auto compute_bwd = [&](BFrags& f, const unsigned char* next, int c) {
        const int cc = nch - 1 - c;
        const int64_t start = t0 + (int64_t)C * cc;
        const int nvalid = (int)min((int64_t)C, t1 - start);
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
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
        if (a.chunk_state) store_state(sb, s0 + cc);
        // the output gradient as a token operand (scale applied to the products)
        bf16xEL dob[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dob[ct][i] = (bf16)f.dov[ct][0][i];
                if constexpr (NB == 2) dob[ct][4 + i] = (bf16)f.dov[ct][NB - 1][i];
            }
        // dU = Kd dS' + scale Aqk^T dO
        floatx4 dU[CT][NB], aux[CT][NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                dU[ct][bb] = zero;
                aux[ct][bb] = mfma_tok(f.aqkt[bb], dob[ct], zero);
            }
        read_blocks(f.aqkt, next, BR::AQKT);
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    dU[ct][bb] = mfma32(f.kd[bb][j], sb[ct][j], dU[ct][bb]);
        read_kd_do(f, next);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) dU[ct][bb][i] += a.scale * aux[ct][bb][i];
        if (a.chunk_u) store_tok(a.chunk_u, dU, s0 + cc);
        bf16xEL duc[CT], yc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                duc[ct][i] = (bf16)dU[ct][0][i];
                if constexpr (NB == 2) duc[ct][4 + i] = (bf16)dU[ct][NB - 1][i];
            }
        // dV = Tb^T dU: the value gradient of the chunk's tokens
        floatx4 dV[CT][NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) dV[ct][bb] = mfma_tok(f.tbt[bb], duc[ct], zero);
        read_blocks(f.tbt, next, BR::TBT);
        if (a.chunk_y) store_tok(a.chunk_y, dV, s0 + cc);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                yc[ct][i] = (bf16)dV[ct][0][i];
                if constexpr (NB == 2) yc[ct][4 + i] = (bf16)dV[ct][NB - 1][i];
            }
        if (a.o) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const u32x4 w = __builtin_bit_cast(u32x4, yc[ct]);
#pragma unroll
                for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * bb + 4 * lg + i, e = 4 * bb + i;
                        if (row < nvalid)
                            a.o[(start + row) * vstride + (int64_t)h * a.V + cb + cw + 16 * ct + lr] =
                                (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                    }
            }
        }
        // dS = Diag(Gam_C) dS' + nKG^T dV + scale QG^T dO
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[ct][t][i] *= f.gc[t][i];
        read_bgc(f, next);
        floatx4 QD[CT][KT];
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) QD[ct][t] = mfma_tok(f.qgt[t], dob[ct], zero);
        read_tiles(f.qgt, next, BR::QGT);
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) S[ct][t] = mfma_tok(f.nkgt[t], yc[ct], S[ct][t]);
        read_tiles(f.nkgt, next, BR::NKGT);
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[ct][t][i] += a.scale * QD[ct][t][i];
    };

    if (nch > 0) {
        __syncthreads();  // chunk 0 is in buffer 0
        int s1b = 1;      // buffer of chunk c + 1: (c + 1) % 2
        if constexpr (BWD) {
            BFrags fr;
            read_kd_do(fr, stage[0]);
            read_tiles(fr.qgt, stage[0], BR::QGT);
            read_tiles(fr.nkgt, stage[0], BR::NKGT);
            read_blocks(fr.tbt, stage[0], BR::TBT);
            read_blocks(fr.aqkt, stage[0], BR::AQKT);
            read_bgc(fr, stage[0]);
            __syncthreads();  // chunk 1 is in buffer 1; buffer 0 may be overwritten
            for (int c = 0; c < nround; ++c) {
                if (c < nch) compute_bwd(fr, stage[s1b], c);  // uniform over the workgroup
                __syncthreads();
                s1b ^= 1;
            }
        } else {
            Frags fr;
            read_nkg_v(fr, stage[0]);
            read_qg(fr, stage[0]);
            read_gc(fr, stage[0]);
            read_tb(fr, stage[0]);
            read_kdt(fr, stage[0]);
            read_aqk(fr, stage[0]);
            __syncthreads();  // chunk 1 is in buffer 1; buffer 0 may be overwritten
            for (int c = 0; c < nround; ++c) {
                if (c < nch) compute(fr, stage[s1b], c);  // uniform over the workgroup
                __syncthreads();
                s1b ^= 1;
            }
        }
    }

    if (trans) {
        float* mo = a.trans_out + ((int64_t)n * a.H + h) * K * K + (cb - a.V) + cw + lr;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    mo[16 * ct + (int64_t)tile_channel(t, 4 * lg + i) * K] = S[ct][t][i];
    } else if (a.final_state) {
        const int nf = a.final_map ? a.final_map[n] : n;
        if (nf >= 0) {
            const int64_t sf = ((int64_t)nf * a.H + h) * K * a.V + cb + cw + lr;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a.final_state[sf + 16 * ct + (int64_t)tile_channel(t, 4 * lg + i) * a.V] =
                            S[ct][t][i];
        }
    }
}

// Compute waves per workgroup, 16-column state tiles per compute wave, loader
// waves, and the loaders' prefetch depth in chunks.  Two compute waves of one
// tile each give 32 value columns per workgroup, so a batch of 64
// sequence-head pairs (4 column blocks each at V = 128) fills every CU; with
// two loader waves there is one wave per SIMD, and the compute waves keep
// every operand of the next chunk in registers.  A CU's pace is set by the
// record bytes it loads per chunk; more columns per workgroup amortise them
// but leave CUs idle unless the grid exceeds the CU count (the wide form
// below).
#ifndef KDA_RECUR_WAVES
#define KDA_RECUR_WAVES 2
#endif
#ifndef KDA_RECUR_TILES
#define KDA_RECUR_TILES 1
#endif
#ifndef KDA_RECUR_LOADERS
#define KDA_RECUR_LOADERS 2
#endif
#ifndef KDA_RECUR_DEPTH
#define KDA_RECUR_DEPTH 4
#endif
// Grids larger than the CU count (forward pass): four compute waves of one
// tile (64 value columns per workgroup) and four loader waves, one workgroup
// per CU.  Each record then serves twice the columns per pass through a CU,
// which beats two 32-column workgroups sharing the CU; with fewer workgroups
// than CUs it leaves CUs idle and is slower.
#ifndef KDA_RECUR_WIDE_WAVES
#define KDA_RECUR_WIDE_WAVES 4
#endif
#ifndef KDA_RECUR_WIDE_LOADERS
#define KDA_RECUR_WIDE_LOADERS 4
#endif
#ifndef KDA_RECUR_WIDE_DEPTH
#define KDA_RECUR_WIDE_DEPTH 2
#endif
constexpr int RECUR_WAVES = KDA_RECUR_WAVES;
constexpr int RECUR_WIDE_WAVES = KDA_RECUR_WIDE_WAVES;
constexpr int RECUR_WIDE_LOADERS = KDA_RECUR_WIDE_LOADERS;
constexpr int RECUR_WIDE_DEPTH = KDA_RECUR_WIDE_DEPTH;
constexpr int RECUR_TILES = KDA_RECUR_TILES;
constexpr int RECUR_LOADERS = KDA_RECUR_LOADERS;
constexpr int RECUR_DEPTH = KDA_RECUR_DEPTH;

// Compute units of the current device (queried once per device).
int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// One workgroup per CU in every mode.  Forward grids beyond the CU count run
// the wide form (64 columns per workgroup); the other modes queue their
// extra workgroups for free CUs (a register budget for two resident per CU
// spilled 60-80 registers in the state-storing modes and was 30% slower).
template <class F>
void launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t stream, const LaunchEvents* ev,
                   const RecurArgs& a) {
    if (ev)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev->start, ev->stop, 0, a);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, a);
}

template <int K, int MODE>
void launch_recur_t(const RecurArgs& a, hipStream_t stream, const LaunchEvents* ev) {
    const int cols = a.V + (a.trans_out ? K : 0);
    const int vs = cols / (16 * RECUR_TILES * RECUR_WAVES);
    const int64_t pairs = (int64_t)a.n_seqs * a.H;
    const int64_t groups = (pairs + 7) / 8;  // the grid covers whole groups of 8 pairs
    if constexpr (MODE == RECUR_FWD) {
        if (pairs * vs > device_cus()) {
            const int vsw = cols / (16 * RECUR_WIDE_WAVES);
            launch_kernel(kda_recur_kernel<K, RECUR_WIDE_WAVES, 1, RECUR_WIDE_LOADERS,
                                           RECUR_WIDE_DEPTH, 1, MODE>,
                          dim3((unsigned)(groups * 8 * vsw)),
                          dim3(64 * (RECUR_WIDE_WAVES + RECUR_WIDE_LOADERS)), stream, ev, a);
            return;
        }
    }
    launch_kernel(kda_recur_kernel<K, RECUR_WAVES, RECUR_TILES, RECUR_LOADERS, RECUR_DEPTH, 1, MODE>,
                  dim3((unsigned)(groups * 8 * vs)), dim3(64 * (RECUR_WAVES + RECUR_LOADERS)),
                  stream, ev, a);
}

template <int K>
void launch_recur_k(const RecurArgs& a, hipStream_t stream, RecurMode mode,
                    const LaunchEvents* ev) {
    if (mode == RECUR_STORE) launch_recur_t<K, RECUR_STORE>(a, stream, ev);
    else if (mode == RECUR_FWD_STORE) launch_recur_t<K, RECUR_FWD_STORE>(a, stream, ev);
    else if (mode == RECUR_BWD) launch_recur_t<K, RECUR_BWD>(a, stream, ev);
    else launch_recur_t<K, RECUR_FWD>(a, stream, ev);
}

void launch_recur(const RecurArgs& a, int K, hipStream_t stream, RecurMode mode,
                  const LaunchEvents* ev) {
    if (K == 128) launch_recur_k<128>(a, stream, mode, ev);
    else launch_recur_k<64>(a, stream, mode, ev);
}

}  // namespace kda
