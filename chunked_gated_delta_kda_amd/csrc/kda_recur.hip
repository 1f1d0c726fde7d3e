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
// transposes and no LDS traffic; the only conversions are fp32 -> bf16 of
// the operand copies.  Record fragments for chunk i+1 are loaded while
// chunk i computes.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

template <int K>
struct Frag {
    static constexpr int KS = K / 32, KT = K / 16;
    bf16x8 nkg[KS];
    bf16x8 qg[KS];
    bf16x4 kdt[KT];
    bf16x4 aqk, tb;
    floatx4 gc[KT];
    uint16_t v[4];
};

template <int K>
__device__ __forceinline__ void load_frag(Frag<K>& f, const unsigned char* rec, int lane, int lg,
                                          const uint16_t* vbase, int64_t vstride, int nvalid) {
    using R = Rec<K>;
#pragma unroll
    for (int j = 0; j < K / 32; ++j) {
        f.nkg[j] = *reinterpret_cast<const bf16x8*>(rec + R::NKG + (j * 64 + lane) * 16);
        f.qg[j] = *reinterpret_cast<const bf16x8*>(rec + R::QG + (j * 64 + lane) * 16);
    }
#pragma unroll
    for (int b = 0; b < K / 16; ++b) {
        f.kdt[b] = *reinterpret_cast<const bf16x4*>(rec + R::KDT + (b * 64 + lane) * 8);
        f.gc[b] = *reinterpret_cast<const floatx4*>(rec + R::GAMC + (16 * b + 4 * lg) * 4);
    }
    f.aqk = *reinterpret_cast<const bf16x4*>(rec + R::AQK + lane * 8);
    f.tb = *reinterpret_cast<const bf16x4*>(rec + R::TB + lane * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * lg + i;
        f.v[i] = t < nvalid ? vbase[t * vstride] : (uint16_t)0;
    }
}

template <int K, int NW>
__global__ __launch_bounds__(64 * NW) void kda_recur_kernel(RecurArgs a) {
    using R = Rec<K>;
    constexpr int KS = K / 32, KT = K / 16;
    const int VS = a.V / (16 * NW);
    const int vs = blockIdx.x % VS;
    const int nh = blockIdx.x / VS;
    const int h = nh % a.H, n = nh / a.H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int c0 = (vs * NW + wave) * 16;  // first value column of this wave

    // state tiles: S[b][i] = S[16 b + 4 lg + i][c0 + lr]
    floatx4 S[KT];
    const int64_t st = ((int64_t)n * a.H + h) * K * a.V + c0 + lr;
#pragma unroll
    for (int b = 0; b < KT; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[b][i] = a.initial_state ? a.initial_state[st + (int64_t)(16 * b + 4 * lg + i) * a.V]
                                      : 0.f;

    const int s0 = a.chunk_off[n], s1 = a.chunk_off[n + 1];
    const int64_t t0 = a.seq_start[n], t1 = a.seq_start[n + 1];
    const int64_t vstride = (int64_t)a.H * a.V;  // between consecutive tokens
    const unsigned char* rec_h = a.rec + (int64_t)h * R::BYTES;
    const int64_t rec_stride = (int64_t)a.H * R::BYTES;

    Frag<K> cur, nxt;
    if (s0 < s1) {
        const int nv = (int)min((int64_t)C, t1 - t0);
        load_frag<K>(cur, rec_h + s0 * rec_stride, lane, lg,
                     a.v + t0 * vstride + (int64_t)h * a.V + c0 + lr, vstride, nv);
    }
    for (int s = s0; s < s1; ++s) {
        const int64_t start = t0 + (int64_t)C * (s - s0);
        const int nvalid = (int)min((int64_t)C, t1 - start);
        if (s + 1 < s1) {
            const int64_t ns = start + C;
            load_frag<K>(nxt, rec_h + (s + 1) * rec_stride, lane, lg,
                         a.v + ns * vstride + (int64_t)h * a.V + c0 + lr, vstride,
                         (int)min((int64_t)C, t1 - ns));
        }
        // bf16 operand copy of the state: k-step j pairs tiles 2j and 2j+1
        bf16x8 sb[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sb[j][e] = (bf16)S[2 * j][e];
                sb[j][4 + e] = (bf16)S[2 * j + 1][e];
            }
        floatx4 Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = bf2f(cur.v[i]);
#pragma unroll
        for (int j = 0; j < KS; ++j) Y = mfma32(cur.nkg[j], sb[j], Y);  // V - KG S
        floatx4 OT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j) OT = mfma32(sb[j], cur.qg[j], OT);  // S^T QG^T
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        const bf16x4 ub = to_bf16x4(mfma16(cur.tb, to_bf16x4(Y), zero));  // U'
        OT = mfma16(ub, cur.aqk, OT);  // + U'^T Aqk^T
        // OT[i] = O[token lr][column c0 + 4 lg + i]
        if (lr < nvalid) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (bf16)(a.scale * OT[i]);
            *reinterpret_cast<bf16x4*>(a.o + (start + lr) * vstride + (int64_t)h * a.V + c0 +
                                       4 * lg) = ov;
        }
#pragma unroll
        for (int b = 0; b < KT; ++b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S[b][i] *= cur.gc[b][i];
            S[b] = mfma16(cur.kdt[b], ub, S[b]);
        }
        if (s + 1 < s1) cur = nxt;
    }

    if (a.final_state) {
#pragma unroll
        for (int b = 0; b < KT; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.final_state[st + (int64_t)(16 * b + 4 * lg + i) * a.V] = S[b][i];
    }
}

// Waves per workgroup: 4 (64 value columns per workgroup).
constexpr int RECUR_WAVES = 4;

template <int K>
void launch_recur_t(const RecurArgs& a, hipStream_t stream) {
    const int vs = a.V / (16 * RECUR_WAVES);
    hipLaunchKernelGGL((kda_recur_kernel<K, RECUR_WAVES>), dim3(a.n_seqs * a.H * vs),
                       dim3(64 * RECUR_WAVES), 0, stream, a);
}

void launch_recur(const RecurArgs& a, int K, hipStream_t stream) {
    if (K == 128) launch_recur_t<128>(a, stream);
    else launch_recur_t<64>(a, stream);
}

}  // namespace kda
