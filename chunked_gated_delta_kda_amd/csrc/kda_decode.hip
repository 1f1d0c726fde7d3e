// kda_decode.hip -- one recurrent step per sequence (gfx950): the single-token
// form of the same recurrence, for decoding after a prefill.
//
// For every (sequence, head), with the state S in [K, V] layout:
//   S' = (I - b k^ k^T) Diag(a) S + b k^ v^T,   o = scale * S'^T q^
// computed as  w = a * S (row scaling),  r = w^T k^,  u = b (v - r),
// S' = w + k^ u^T,  o = scale * S'^T q^.  This is the token recurrence the
// chunked kernels implement, one token at a time; the cuLA pages list decode
// kernels on their inference roadmap (cuLA blog, section "Status &
// Roadmap"; cuLA README, roadmap list), and FlashKDA's parameter table
// (discuss.pytorch.kr, section "FlashKDA의 KDA 연산 구조") fixes the gate,
// beta and norm definitions shared with the forward pass.
//
// The step is bound by HBM: the state is read and written once (2 K V 4
// bytes per pair), everything else is K- or V-sized.  One workgroup per
// (sequence, head, 64 value columns); thread (rg, cq) owns rows
// RPT rg .. RPT rg + RPT - 1 and columns 4 cq .. 4 cq + 3 of the block, so a
// row of the block is 16 threads x 16 bytes, one coalesced 256-byte access.
// Reductions over rows go through LDS.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int DEC_COLS = 64;                 // value columns per workgroup
constexpr int DEC_CQ = DEC_COLS / 4;         // column quads (16)
constexpr int DEC_THREADS = 256;
constexpr int DEC_RG = DEC_THREADS / DEC_CQ;  // row groups (16)

__device__ __forceinline__ void unpack8f(u32x4 v, float* f) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f[2 * u] = bf2f(v[u] & 0xffff);
        f[2 * u + 1] = bf2f(v[u] >> 16);
    }
}

// Loads RPT consecutive bf16 channels starting at channel c0 (RPT = 4 or 8).
template <int RPT>
__device__ __forceinline__ void load_ch(const uint16_t* p, float* f) {
    if constexpr (RPT == 8) {
        unpack8f(*reinterpret_cast<const u32x4*>(p), f);
    } else {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        f[0] = bf2f(w.x & 0xffff);
        f[1] = bf2f(w.x >> 16);
        f[2] = bf2f(w.y & 0xffff);
        f[3] = bf2f(w.y >> 16);
    }
}

}  // namespace

template <int K, bool GDN>
__global__ __launch_bounds__(DEC_THREADS) void kda_decode_kernel(DecodeArgs a) {
    constexpr int RPT = K / DEC_RG;  // rows per thread (8 at K = 128)
    __shared__ float red[DEC_RG][DEC_COLS];
    __shared__ float nrm[2][DEC_RG];

    const int VB = a.V / DEC_COLS;
    const int pair = blockIdx.x / VB, vb = blockIdx.x % VB;
    const int h = pair % a.H;
    const int tid = threadIdx.x;
    const int cq = tid % DEC_CQ, rg = tid / DEC_CQ;
    const int r0 = RPT * rg;                 // first row (channel) of this thread
    const int c0 = vb * DEC_COLS + 4 * cq;   // first value column of this thread
    const int64_t tok = (int64_t)pair;       // row of the [N, H, *] token tensors

    // ---- this thread's channels of q, k and the gate
    float qv[RPT], kv[RPT], la[RPT];
    load_ch<RPT>(a.q + tok * K + r0, qv);
    load_ch<RPT>(a.k + tok * K + r0, kv);
    if constexpr (GDN) {
        const float gl = a.g_gdn[tok];  // log decay, the same for every channel
#pragma unroll
        for (int i = 0; i < RPT; ++i) la[i] = gl;
    } else {
        float gv[RPT];
        load_ch<RPT>(a.g_kda + tok * K + r0, gv);
        const float rate = exp2_hw(a.A_log[h] * LOG2E);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            la[i] = fmaxf(a.lower_bound, -rate * softplus_f(gv[i] + a.dt_bias[(int64_t)h * K + r0 + i]));
    }
    const float braw = bf2f(a.beta[tok]);
    const float b = GDN ? braw : sigmoid_f(braw);

    // ---- the state block, read once (zeros when there is no input state)
    floatx4 S[RPT];
    const int64_t sbase = (int64_t)pair * K * a.V + c0;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        S[i] = a.state_in
                   ? *reinterpret_cast<const floatx4*>(a.state_in + sbase + (int64_t)(r0 + i) * a.V)
                   : zero;
    }

    // ---- L2 norms of q and k over all K channels
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) { sq += qv[i] * qv[i]; sk += kv[i] * kv[i]; }
    if (cq == 0) { nrm[0][rg] = sq; nrm[1][rg] = sk; }
    __syncthreads();
    sq = 0.f;
    sk = 0.f;
#pragma unroll
    for (int j = 0; j < DEC_RG; ++j) { sq += nrm[0][j]; sk += nrm[1][j]; }
    const float iq = rsq_hw(sq + NORM_EPS), ik = rsq_hw(sk + NORM_EPS);

    // ---- w = Diag(a) S;  r = w^T k^  (partial over this thread's rows)
    floatx4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float al = exp2_hw(la[i] * LOG2E), kh = kv[i] * ik;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            S[i][e] *= al;
            r[e] += S[i][e] * kh;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) red[rg][4 * cq + e] = r[e];
    __syncthreads();
    floatx4 u;
    {
        float vv[4];
        const uint2 w = *reinterpret_cast<const uint2*>(a.v + tok * a.V + c0);
        vv[0] = bf2f(w.x & 0xffff);
        vv[1] = bf2f(w.x >> 16);
        vv[2] = bf2f(w.y & 0xffff);
        vv[3] = bf2f(w.y >> 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float rs = 0.f;
#pragma unroll
            for (int j = 0; j < DEC_RG; ++j) rs += red[j][4 * cq + e];
            u[e] = b * (vv[e] - rs);
        }
    }
    __syncthreads();  // red is reused below

    // ---- S' = w + k^ u^T, stored; o = scale S'^T q^ (partial over rows)
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kh = kv[i] * ik, qh = qv[i] * iq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            S[i][e] += kh * u[e];
            o[e] += S[i][e] * qh;
        }
        *reinterpret_cast<floatx4*>(a.state_out + sbase + (int64_t)(r0 + i) * a.V) = S[i];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) red[rg][4 * cq + e] = o[e];
    __syncthreads();
    if (rg == 0) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float os = 0.f;
#pragma unroll
            for (int j = 0; j < DEC_RG; ++j) os += red[j][4 * cq + e];
            ov[e] = (bf16)(a.scale * os);
        }
        *reinterpret_cast<bf16x4*>(a.o + tok * a.V + c0) = ov;
    }
}

template <int K, bool GDN>
void launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.n_pairs * (a.V / DEC_COLS);
    hipLaunchKernelGGL((kda_decode_kernel<K, GDN>), dim3((unsigned)blocks), dim3(DEC_THREADS), 0,
                       stream, a);
}

void launch_decode(const DecodeArgs& a, int K, bool gdn, hipStream_t stream) {
    if (K == 128) {
        if (gdn) launch_decode_t<128, true>(a, stream);
        else launch_decode_t<128, false>(a, stream);
    } else {
        if (gdn) launch_decode_t<64, true>(a, stream);
        else launch_decode_t<64, false>(a, stream);
    }
}

}  // namespace kda
