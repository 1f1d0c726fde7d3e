// kda_bwd.hip -- the backward pass (gfx950): the chunk-parallel gradient
// kernel and the reduction of the gate-parameter gradients (the reverse-pass
// record comes from kda_prep, the two sweeps from kda_recur).
//
// The pages show the backward only as autograd over the forward call (cuLA
// README mirror, section "Usage": o.backward(do) with q, k, v requiring
// grad; the cuLA roadmap lists backward kernels for training, and the
// FlashQLA summary (section "핵심 기능") a backward path beside the forward
// one).  This is the reverse-mode derivative of the chunkwise forward pass
// (kda_recur.hip), chunk by chunk.  Per chunk, with h the state entering it,
// S' = Diag(Gam_C) h + Kd^T U' the state leaving it, U' = Tb Z,
// Z = V - KG h, Tb = T diag(b), T = (I + diag(b) P)^-1,
// P = tril_strict(KG Kinv^T), Kinv = k^ / Gam, O = scale (QG h + Aqk U'),
// Aqk = tril(QG Kinv^T), and dS' the gradient reaching S':
//   dU  = Kd dS' + scale Aqk^T dO          dV  = Tb^T dU
//   dh  = Diag(Gam_C) dS' + scale QG^T dO - KG^T dV
// (the reverse recurrence, kda_recur in its reverse mode), and locally
//   W1 = T^T dU,  dM = scale tril(dO U'^T),  dP = -diag(b) tril_strict(W1 U'^T)
//   db = rowdot(W1, Z) - rowsum(P * (W1 U'^T))
//   dq^ = Gam * (scale dO h^T) + sum_j dM[r,j] k^_j Gam_r / Gam_j
//   dk^ = -Gam * (dV h^T) + sum_j dP[r,j] k^_j Gam_r / Gam_j        (via KG)
//       + sum_r (dM[r,j] q^_r + dP[r,j] k^_r) Gam_r / Gam_j         (via Kinv)
//       + (Gam_C / Gam) * (U' dS'^T)                                (via Kd)
//   dG  = q^ dq^ + k^ (dk^_KG - dk^_Kinv - dk^_Kd), plus, on the chunk's
//         last token, sum_j k^_j dk^_Kd,j + Gam_C * rowsum(h * dS')
//   d log a_t = sum over the chunk's tokens s >= t of dG_s
// followed by the chain rule through the L2 norms, the gate and the sigmoid.
// Every ratio Gam_r / Gam_j (r >= j) is formed from two factors of the same
// 16-token block, or from factors that are both <= 1 across the two blocks,
// as in the forward pass.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

// ------------------------------------------------------------ gradient kernel
namespace {

constexpr int ROW_SHR1 = 0x111, ROW_SHR2 = 0x112, ROW_SHR4 = 0x114, ROW_SHR8 = 0x118;

__device__ __forceinline__ float row_scan16(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, ROW_SHR1, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, ROW_SHR2, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, ROW_SHR4, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, ROW_SHR8, 0xf, 0xf, false);
    return x;
}
// sum over the 16 lanes of a row (every lane gets it)
__device__ __forceinline__ float row_sum16(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f[2 * u] = bf2f(v[u] & 0xffff);
        f[2 * u + 1] = bf2f(v[u] >> 16);
    }
}

__device__ __forceinline__ bf16x8 pack8(const float* f) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)f[e];
    return r;
}

__device__ __forceinline__ uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, (bf16)x); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): about 16 significant bits
template <class A>
__device__ __forceinline__ void put_split(A& arr, int part, int c, int p, float x) {
    const bf16 hi = (bf16)x;
    arr[0][part][c][p] = __builtin_bit_cast(uint16_t, hi);
    arr[1][part][c][p] = bits(x - (float)hi);
}

}  // namespace

// One workgroup per (chunk slot, head) and 2 K / 32 waves: wave w owns the
// 16-token block b = w % 2 and the channel group q = w / 2 of 32 channels.
// Lane l = m + 16 g of a wave owns token 16 b + m and the channels
// 32 q + 8 g + e, e < 8 (the row layout of kda_prep, one k-step per wave).
// Products that contract over channels read their operands from registers
// (partial sums over the channel groups meet in LDS); products that contract over
// tokens read token-ordered copies from LDS; products that contract over
// value columns read the stored states and [C, V] rows.  Every result that is
// a function of (token, channel) is produced transposed (channels as MFMA rows
// in the tile_channel order), which lands it in the owner lane's registers.
// Swizzle key of state row (channel) ch, over PR pieces per row: bits 0-1 and
// 3-4 of the channel, which take 16 distinct values over a state tile's rows.
template <int PR>
__device__ __forceinline__ int st_key(int ch) {
    return ((((ch >> 3) & 3) << 2) | (ch & 3)) & (PR - 1);
}

template <int K, int V, bool GDN>
__global__ __launch_bounds__(4 * K) void kda_bwd_chunk_kernel(BwdArgs a) {
    static_assert(NB == 2, "the gradient kernel assumes 32-token chunks");
    constexpr int KS = K / 32, KH = 1, KT = K / 16, VS = V / 32, VT = V / 16;
    constexpr int NQ = KS;             // channel groups (waves per token block)
    constexpr int NT = 128 * NQ;       // threads
    static_assert(VT % NQ == 0, "value tiles are dealt evenly to the channel groups");
    constexpr int UP = V + 8;  // padded row of the U' / W1 copies (bf16)
    using R = Rec<K>;
    // LDS, 155 KB at K = V = 128 (one workgroup per CU, as the registers
    // allow): regions whose lifetimes do not overlap share memory (the phase
    // of each is noted); the state copies have a region of their own.
    constexpr int OFF_GEND = 0;                               // float [2][K], all phases
    constexpr int OFF_BETA = OFF_GEND + 2 * K * 4;            // float [C], until dM
    constexpr int OFF_P = OFF_BETA + C * 4;                   // float [NQ][C][C+1], P .. dM
    constexpr int OFF_XT = OFF_P + NQ * C * (C + 1) * 4;      // bf16 [2][3][K][C], P .. intra
    constexpr int OFF_U = OFF_XT + 2 * 3 * K * C * 2;         // bf16 [C][UP], U' .. V-products
    constexpr int OFF_W = OFF_U + C * UP * 2;                 // bf16 [C][UP], U' .. dM;
                                                              //   then the late sums below
    constexpr int OFF_DM = OFF_W + C * UP * 2;                // bf16 4 x [C][C], dM .. intra;
                                                              //   before: kbc0, norms
    constexpr int OFF_DB = OFF_DM + 4 * C * C * 2;            // float [NQ][C], dM .. end
    // the chunk's entering state h and dL/d(leaving state), bf16 [K][V] each,
    // copied in by the DMA engine while the earlier phases run.  Each row's
    // 16-byte pieces are stored XOR-swizzled by a key taken from the channel
    // bits that differ between the 16 rows of a state tile, so a tile read
    // spreads over the banks.
    constexpr int OFF_ST = (OFF_DB + NQ * C * 4 + 15) / 16 * 16;
    constexpr int PR = V / 8;                    // 16-byte pieces per state row
    constexpr int ST_PPT = 2 * K * PR / NT;      // pieces per thread
    static_assert(2 * K * PR % NT == 0, "state pieces are dealt evenly");
    constexpr int LDS_BYTES = OFF_ST + 2 * K * V * 2;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS per workgroup");
    static_assert(KS * 64 * 16 + NQ * C * 2 * 4 <= 4 * C * C * 2, "early region");
    static_assert(6 * K * 4 + NQ * C * 2 * 4 + 2 * NQ * 4 <= C * UP * 2, "late region");

    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
    auto& gend_s = *reinterpret_cast<float(*)[2][K]>(smem + OFF_GEND);
    auto& beta_s = *reinterpret_cast<float(*)[C]>(smem + OFF_BETA);
    // tril_strict(KG Kinv^T) as the channel groups' shares: P = sum over q of
    // P_s[q], added in the order q = 0, 1, .. wherever P is read
    auto& P_s = *reinterpret_cast<float(*)[NQ][C][C + 1]>(smem + OFF_P);
    auto P_at = [&](int r, int col) {
        float sum = P_s[0][r][col];
#pragma unroll
        for (int qq = 1; qq < NQ; ++qq) sum += P_s[qq][r][col];
        return sum;
    };
    // channel-major token operands [hi/lo][part][c][pos(s)]: 0: k^ 2^-Gl,
    // 1: q^ 2^Gl, 2: k^ 2^Gl (Gl: log2 decay within the token's block), each as
    // a bf16 pair hi + lo.  A token pair (r, j) enters dG_r through one operand
    // and dG_j, with the opposite sign, through another; in the reverse
    // cumulative sum over the chunk the two cancel exactly unless their
    // roundings differ, so these operands carry ~16 significant bits.
    auto& xt_s = *reinterpret_cast<uint16_t(*)[2][3][K][C]>(smem + OFF_XT);
    auto& u_s = *reinterpret_cast<uint16_t(*)[C][UP]>(smem + OFF_U);  // U' rows
    auto& w_s = *reinterpret_cast<uint16_t(*)[C][UP]>(smem + OFF_W);  // W1 rows
    auto& dmr_s = *reinterpret_cast<uint16_t(*)[C][C]>(smem + OFF_DM);              // [r][pos(j)]
    auto& dmc_s = *reinterpret_cast<uint16_t(*)[C][C]>(smem + OFF_DM + C * C * 2);  // [j][pos(r)]
    auto& dpr_s = *reinterpret_cast<uint16_t(*)[C][C]>(smem + OFF_DM + 2 * C * C * 2);
    auto& dpc_s = *reinterpret_cast<uint16_t(*)[C][C]>(smem + OFF_DM + 3 * C * C * 2);
    // early tenants of the dM region
    auto& kbc0_s = *reinterpret_cast<bf16x8(*)[KS * 64]>(smem + OFF_DM);  // block 0: k^ 2^(G_end0 - G)
    auto& nrm_s = *reinterpret_cast<float(*)[NQ][C][2]>(smem + OFF_DM + KS * 64 * 16);
    auto& dbeta_s = *reinterpret_cast<float(*)[NQ][C]>(smem + OFF_DB);  // per channel group
    // late tenants of the W1 region
    auto& kd_s = *reinterpret_cast<float(*)[2][K]>(smem + OFF_W);  // per block: sum of k^ dk^_Kd
    auto& hs_s = *reinterpret_cast<float(*)[K]>(smem + OFF_W + 2 * K * 4);  // rowsum(h * dS')
    auto& tot_s = *reinterpret_cast<float(*)[K]>(smem + OFF_W + 3 * K * 4);  // block 1's dG totals
    auto& dot_s = *reinterpret_cast<float(*)[NQ][C][2]>(smem + OFF_W + 4 * K * 4);
    auto& red_s = *reinterpret_cast<float(*)[2][K]>(smem + OFF_W + 4 * K * 4 + NQ * C * 2 * 4);
    auto& alog_s = *reinterpret_cast<float(*)[2 * NQ]>(smem + OFF_W + 6 * K * 4 + NQ * C * 2 * 4);

    // heads fastest: the workgroups in flight together read and write whole
    // token rows ([H, K] contiguous) and consecutive chunk states
    const int slot = blockIdx.x / a.H;
    const int h = blockIdx.x % a.H;
    const int wave = threadIdx.x >> 6;
    const int blk = wave & 1, hf = wave >> 1;  // token block, channel group
    const int L = threadIdx.x & 63, m = L & 15, g = L >> 4;
    const int j0 = hf;  // this wave's k-step (channels 32 j0 ..)

    int n;
    if (!a.packed) {
        n = slot / ((a.T + C - 1) / C);
        if (n >= a.n_seqs) return;
    } else {
        if (slot >= a.chunk_off[a.n_seqs]) {
            // a slot past the packed chunks (the grid covers their upper bound):
            // its share of the gate-parameter sums is zero
            if constexpr (!GDN) {
                const int64_t chb = (int64_t)slot * a.H + h;
                for (int c = threadIdx.x; c < K; c += NT) a.part_dt[chb * K + c] = 0.f;
                if (threadIdx.x == 0) a.part_alog[chb] = 0.f;
            }
            return;
        }
        int lo = 0, hi = a.n_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.chunk_off[mid] <= slot) lo = mid; else hi = mid;
        }
        n = lo;
    }
    int64_t t0, t1;
    int s0, s1;
    seq_span(a, n, t0, t1, s0, s1);
    const int64_t start = t0 + (int64_t)C * (slot - s0);
    const int nvalid = (int)min((int64_t)C, t1 - start);
    const int row = 16 * blk + m;
    const bool valid = row < nvalid;
    const int64_t lrow = (start + (valid ? row : 0)) * a.H + h;
    const int64_t ch_base = (int64_t)slot * a.H + h;  // chunk-head index of the stored tensors

    // start the copies of h and dS' into LDS; they land while the phases
    // below run and are waited for before the products over value columns
    {
        const int nw = NT / 64;
#pragma unroll
        for (int i = 0; i < ST_PPT; ++i) {
            const int j = i * nw + wave;                 // 1 KB block of the LDS copy
            const int pc = 64 * j + L;                   // this lane's piece
            const int arr = pc / (K * PR), pp = pc % (K * PR);
            const int r = pp / PR, sl = pp % PR;
            const uint16_t* src = (arr ? a.dss : a.hs) + ch_base * K * V + (int64_t)r * V +
                                  8 * (sl ^ st_key<PR>(r));
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void*)(smem + OFF_ST + 1024 * j), 16, 0, 0);
        }
    }

    // ---- this lane's row and channels: q^, k^, log2 decay; beta
    float qh[KH][8], kh[KH][8], G[KH][8];
    float xg[KH][8];  // KDA: the gate's pre-activation g + dt_bias, kept for the chain rule
    {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int jj = 0; jj < KH; ++jj) {
            const int c = 32 * (j0 + jj) + 8 * g;
            unpack8(*reinterpret_cast<const u32x4*>(a.q + lrow * K + c), qh[jj]);
            unpack8(*reinterpret_cast<const u32x4*>(a.k + lrow * K + c), kh[jj]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (!valid) { qh[jj][e] = 0.f; kh[jj][e] = 0.f; }
                sq += qh[jj][e] * qh[jj][e];
                sk += kh[jj][e] * kh[jj][e];
            }
        }
        sq += __shfl_xor(sq, 16, 64);
        sq += __shfl_xor(sq, 32, 64);
        sk += __shfl_xor(sk, 16, 64);
        sk += __shfl_xor(sk, 32, 64);
        if (g == 0) { nrm_s[hf][row][0] = sq; nrm_s[hf][row][1] = sk; }
    }
    const float braw = bf2f(a.beta[lrow]);
    const float b = valid ? (GDN ? braw : sigmoid_f(braw)) : 0.f;
    const float rate = GDN ? 0.f : exp2_hw(a.A_log[h] * LOG2E);
    if constexpr (GDN) {
        const float la = valid ? a.g_gdn[lrow] * LOG2E : 0.f;
#pragma unroll
        for (int jj = 0; jj < KH; ++jj)
#pragma unroll
            for (int e = 0; e < 8; ++e) G[jj][e] = la;
    } else {
#pragma unroll
        for (int jj = 0; jj < KH; ++jj) {
            const int c = 32 * (j0 + jj) + 8 * g;
            float x[8];
            unpack8(*reinterpret_cast<const u32x4*>(a.g_kda + lrow * K + c), x);
            const floatx4 d0 = *reinterpret_cast<const floatx4*>(a.dt_bias + (int64_t)h * K + c);
            const floatx4 d1 = *reinterpret_cast<const floatx4*>(a.dt_bias + (int64_t)h * K + c + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xg[jj][e] = x[e] + (e < 4 ? d0[e] : d1[e - 4]);
                // every row (padding rows re-read a real row; the value is
                // finite) and zeroed on padding rows: no branch per element
                G[jj][e] = fmaxf(a.lower_bound, -rate * softplus_f(xg[jj][e])) * LOG2E *
                           (valid ? 1.f : 0.f);
            }
        }
    }
    // in-block inclusive prefix (log2), block totals to LDS
#pragma unroll
    for (int jj = 0; jj < KH; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            G[jj][e] = row_scan16(G[jj][e]);
            if (m == 15) gend_s[blk][32 * (j0 + jj) + 8 * g + e] = G[jj][e];
        }
    if (hf == 0 && g == 0) beta_s[row] = b;
    __syncthreads();
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) { sq += nrm_s[qq][row][0]; sk += nrm_s[qq][row][1]; }
    const float iq = rsq_hw(sq + NORM_EPS), ik = rsq_hw(sk + NORM_EPS);
#pragma unroll
    for (int jj = 0; jj < KH; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) { qh[jj][e] *= iq; kh[jj][e] *= ik; }

    // ---- decay-weighted operands; this half's share of P; token-ordered copies
    floatx4 Pacc = {0.f, 0.f, 0.f, 0.f};
    bf16x8 ka_f[KH];
#pragma unroll
    for (int jj = 0; jj < KH; ++jj) {
        float ka[8], kbs[8], kbc[8], qa[8];
        const int p = tok_pos(row);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 32 * (j0 + jj) + 8 * g + e;
            const float ga = exp2_hw(G[jj][e]);
            ka[e] = kh[jj][e] * ga;
            qa[e] = qh[jj][e] * ga;
            kbs[e] = kh[jj][e] * exp2_hw(-G[jj][e]);
            kbc[e] = kh[jj][e] * exp2_hw(gend_s[0][c] - G[jj][e]);  // used for block 0 only
            put_split(xt_s, 0, c, p, kbs[e]);
            put_split(xt_s, 1, c, p, qa[e]);
            put_split(xt_s, 2, c, p, ka[e]);
        }
        ka_f[jj] = pack8(ka);
        Pacc = mfma32(ka_f[jj], pack8(kbs), Pacc);  // P[16b + 4g' + i][16b + n], this half
        if (blk == 0) kbc0_s[(j0 + jj) * 64 + L] = pack8(kbc);
    }
    __syncthreads();
    {
        // lane (n, g') of the D layout: rows 4 g' + i, column n (= m here)
        floatx4 Pc = {0.f, 0.f, 0.f, 0.f};
        if (blk == 1) {
#pragma unroll
            for (int jj = 0; jj < KH; ++jj) Pc = mfma32(ka_f[jj], kbc0_s[(j0 + jj) * 64 + L], Pc);
        }
        // each channel group's share into a slot of its own; readers add the
        // shares in a fixed order, so the sum is reproducible
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * blk + 4 * g + i;
            P_s[hf][r][16 * blk + m] = (m < 4 * g + i) ? Pacc[i] : 0.f;
            P_s[hf][r][16 * (1 - blk) + m] = blk == 1 ? Pc[i] : 0.f;
        }
    }
    __syncthreads();

    // ---- U' = Tb Z and W1 = T^T dU for this block's rows and this half's value
    // tiles (D layout); rowdot(W1, Z) on the way.  W1 needs no inverse:
    // (I + diag(b) P)^T W1 = dU and diag(b) W1 = Tb^T dU = dV give
    // W1 = dU - P^T dV.
    float zw[4] = {0.f, 0.f, 0.f, 0.f};
    {
        const bf16xEL tb = *reinterpret_cast<const bf16xEL*>(
            a.rec + ch_base * R::BYTES + R::TB + (blk * 64 + L) * (2 * EL));
        // P^T rows of this block as a token operand: slot (g, e) holds P[tok(g, e)][16 b + m]
        float ptf[EL];
#pragma unroll
        for (int e = 0; e < EL; ++e) ptf[e] = P_at(16 * (e >> 2) + 4 * g + (e & 3), 16 * blk + m);
        const bf16xEL apt = pack8(ptf);
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int vv = 0; vv < VT / NQ; ++vv) {
            const int col = 16 * (hf * (VT / NQ) + vv) + m;
            const int64_t cbase = (ch_base * V + col) * C;
            const u32x4 wz = *reinterpret_cast<const u32x4*>(a.zt + cbase + EL * g);
            const bf16xEL bz = __builtin_bit_cast(bf16xEL, wz);
            const bf16xEL by = *reinterpret_cast<const bf16xEL*>(a.yt + cbase + EL * g);
            // dU in D layout: rows 16 b + 4 g + i sit at positions EL g + 4 b + i
            const uint2 wdu = *reinterpret_cast<const uint2*>(a.dut + cbase + EL * g + 4 * blk);
            const floatx4 U = mfma_tok(tb, bz, zero);
            const floatx4 PY = mfma_tok(apt, by, zero);
            const float duf[4] = {bf2f(wdu.x & 0xffff), bf2f(wdu.x >> 16), bf2f(wdu.y & 0xffff),
                                  bf2f(wdu.y >> 16)};
            float zf[8];
            unpack8(wz, zf);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float Wi = duf[i] - PY[i];
                zw[i] += Wi * zf[4 * blk + i];  // Z[16b + 4g + i][col]
                u_s[16 * blk + 4 * g + i][col] = bits(U[i]);
                w_s[16 * blk + 4 * g + i][col] = bits(Wi);
            }
        }
    }
    __syncthreads();

    // ---- dM = scale tril(dO U'^T), E1 = W1 U'^T, dP for this block's rows and
    // the 16 columns cb = q (channel groups 0 and 1); db's share
    bf16x8 dof[VS];
#pragma unroll
    for (int jv = 0; jv < VS; ++jv) {
        const u32x4 zero4 = {0u, 0u, 0u, 0u};
        const u32x4 x = *reinterpret_cast<const u32x4*>(a.d_o + lrow * V + 32 * jv + 8 * g);
        dof[jv] = __builtin_bit_cast(bf16x8, valid ? x : zero4);
    }
    {
        const int cb = hf;
        float dbp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dbp[i] = zw[i];
        if (cb < 2) {
        floatx4 dm = {0.f, 0.f, 0.f, 0.f}, e1 = dm;
#pragma unroll
        for (int jv = 0; jv < VS; ++jv) {
            const bf16x8 bu = *reinterpret_cast<const bf16x8*>(&u_s[16 * cb + m][32 * jv + 8 * g]);
            const bf16x8 aw = *reinterpret_cast<const bf16x8*>(&w_s[16 * blk + m][32 * jv + 8 * g]);
            dm = mfma32(dof[jv], bu, dm);
            e1 = mfma32(aw, bu, e1);
        }
        const int j = 16 * cb + m;  // this lane's column
        bf16x4 dmv, dpv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * blk + 4 * g + i;
            const float dmx = j <= r ? a.scale * dm[i] : 0.f;
            const float dpx = j < r ? -beta_s[r] * e1[i] : 0.f;
            // read for every lane (in range) and masked by a factor, so the
            // four rows' reads are issued together instead of one branch each
            dbp[i] -= P_at(r, j) * e1[i] * (j < r ? 1.f : 0.f);
            dmr_s[r][tok_pos(j)] = bits(dmx);
            dpr_s[r][tok_pos(j)] = bits(dpx);
            dmv[i] = (bf16)dmx;
            dpv[i] = (bf16)dpx;
        }
        // [j][pos(r)]: rows 16 b + 4 g + i sit at positions EL g + 4 b + i
        *reinterpret_cast<bf16x4*>(&dmc_s[j][EL * g + 4 * blk]) = dmv;
        *reinterpret_cast<bf16x4*>(&dpc_s[j][EL * g + 4 * blk]) = dpv;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = row_sum16(dbp[i]);
            if (m == 0) dbeta_s[hf][16 * blk + 4 * g + i] = s;
        }
    }
    __syncthreads();

    // ---- per-channel accumulators of this lane's row
    float dqh[KH][8], dkh[KH][8], dks[KH][8];  // dq^, dk^, dk^_KG - dk^_Kinv - dk^_Kd
#pragma unroll
    for (int jj = 0; jj < KH; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) { dqh[jj][e] = 0.f; dkh[jj][e] = 0.f; dks[jj][e] = 0.f; }

    // intra-chunk products over tokens; result tile t holds channels
    // rho(t, 4 g + i) = 32 (t / 2) + 8 g + 4 (t % 2) + i of row 16 b + m
    {
        // (operands are split and joined as 32-bit words: element-wise moves
        // inside bf16 vectors are avoided, see kda_recur.hip)
        const u32x4 wmr = *reinterpret_cast<const u32x4*>(&dmr_s[16 * blk + m][EL * g]);
        const u32x4 wpr = *reinterpret_cast<const u32x4*>(&dpr_s[16 * blk + m][EL * g]);
        u32x4 wmc = *reinterpret_cast<const u32x4*>(&dmc_s[16 * blk + m][EL * g]);
        u32x4 wpc = *reinterpret_cast<const u32x4*>(&dpc_s[16 * blk + m][EL * g]);
        // token slots 0..3 hold block 0, slots 4..7 block 1.  Block 1's rows r
        // reach block 0's tokens j through 2^(G_end0 - Gl_j) = 2^G_end0 2^-Gl_j:
        // those slots are summed apart and scaled by 2^G_end0 per channel.
        u32x4 wmr0 = wmr, wmr1 = wmr, wpr0 = wpr, wpr1 = wpr;
        wmr0[2] = wmr0[3] = wpr0[2] = wpr0[3] = 0u;
        wmr1[0] = wmr1[1] = wpr1[0] = wpr1[1] = 0u;
        // block 0's columns j: rows r of block 0 (same factor) and of block 1
        // (cross factor) summed apart
        u32x4 wmc1 = wmc, wpc1 = wpc;
        if (blk == 0) {
            wmc[2] = wmc[3] = wpc[2] = wpc[3] = 0u;
            wmc1[0] = wmc1[1] = wpc1[0] = wpc1[1] = 0u;
        }
        const bf16xEL bmr0 = __builtin_bit_cast(bf16xEL, wmr0), bmr1 = __builtin_bit_cast(bf16xEL, wmr1);
        const bf16xEL bpr0 = __builtin_bit_cast(bf16xEL, wpr0), bpr1 = __builtin_bit_cast(bf16xEL, wpr1);
        const bf16xEL bmc = __builtin_bit_cast(bf16xEL, wmc), bpc = __builtin_bit_cast(bf16xEL, wpc);
        const bf16xEL bmc1 = __builtin_bit_cast(bf16xEL, wmc1),
                      bpc1 = __builtin_bit_cast(bf16xEL, wpc1);
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt2 = 0; tt2 < 2 * KH; ++tt2) {
            const int t = 2 * j0 + tt2;
            const int ch = tile_channel(t, m);  // this lane's A-operand row
            floatx4 iq0 = zero, iq1 = zero, ik0 = zero, ik1 = zero, ki0 = zero, ki1 = zero;
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {  // hi and lo parts of the operands
                const bf16xEL akb = *reinterpret_cast<const bf16xEL*>(&xt_s[hl][0][ch][EL * g]);
                const bf16xEL aqa = *reinterpret_cast<const bf16xEL*>(&xt_s[hl][1][ch][EL * g]);
                const bf16xEL aka = *reinterpret_cast<const bf16xEL*>(&xt_s[hl][2][ch][EL * g]);
                iq0 = mfma_tok(akb, bmr0, iq0);
                ik0 = mfma_tok(akb, bpr0, ik0);
                if (blk == 1) {
                    iq1 = mfma_tok(akb, bmr1, iq1);
                    ik1 = mfma_tok(akb, bpr1, ik1);
                }
                ki0 = mfma_tok(aka, bpc, mfma_tok(aqa, bmc, ki0));
                if (blk == 0) ki1 = mfma_tok(aka, bpc1, mfma_tok(aqa, bmc1, ki1));
            }
            const int jj = (t >> 1) - j0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * (t & 1) + i;
                const int c = 32 * (j0 + jj) + 8 * g + e;
                const float Gl = G[jj][e];
                const float ga = exp2_hw(Gl);
                // block 1: block-0 tokens carry 2^G_end0; block 0: only block-0 tokens
                const float x0 = blk == 1 ? exp2_hw(gend_s[0][c]) : 1.f;
                const float iq = blk == 1 ? x0 * iq0[i] + iq1[i] : iq0[i];
                const float ik = blk == 1 ? x0 * ik0[i] + ik1[i] : ik0[i];
                const float kinv = blk == 0 ? exp2_hw(-Gl) * ki0[i] + exp2_hw(gend_s[0][c] - Gl) * ki1[i]
                                            : exp2_hw(-Gl) * ki0[i];
                dqh[jj][e] += ga * iq;
                const float dkg = ga * ik;
                dkh[jj][e] += dkg + kinv;
                dks[jj][e] += dkg - kinv;
            }
        }
    }

    // ---- products over value columns with the stored states: dO h^T, dV h^T,
    // U' dS'^T (transposed), and rowsum(h * dS'), for this half's channels
    {
        bf16x8 dvf[VS], uf[VS];
#pragma unroll
        for (int jv = 0; jv < VS; ++jv) {
            const u32x4 zero4 = {0u, 0u, 0u, 0u};
            const u32x4 x = *reinterpret_cast<const u32x4*>(a.dv + lrow * V + 32 * jv + 8 * g);
            dvf[jv] = __builtin_bit_cast(bf16x8, valid ? x : zero4);
            uf[jv] = *reinterpret_cast<const bf16x8*>(&u_s[16 * blk + m][32 * jv + 8 * g]);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's state copies
        __syncthreads();                                   // everyone's
        const unsigned char* st_s = smem + OFF_ST;
#pragma unroll
        for (int tt2 = 0; tt2 < 2 * KH; ++tt2) {
            const int t = 2 * j0 + tt2;
            const int ch = tile_channel(t, m);
            floatx4 hq = {0.f, 0.f, 0.f, 0.f}, hk = hq, hd = hq;
            float hsp = 0.f;
#pragma unroll
            for (int jv = 0; jv < VS; ++jv) {
                const int so = ch * (V * 2) + (((4 * jv + g) ^ st_key<PR>(ch)) << 4);
                const u32x4 wh = *reinterpret_cast<const u32x4*>(st_s + so);
                const u32x4 wd = *reinterpret_cast<const u32x4*>(st_s + K * V * 2 + so);
                const bf16x8 ah = __builtin_bit_cast(bf16x8, wh), ad = __builtin_bit_cast(bf16x8, wd);
                hq = mfma32(ah, dof[jv], hq);
                hk = mfma32(ah, dvf[jv], hk);
                hd = mfma32(ad, uf[jv], hd);
                float fh[8], fd[8];
                unpack8(wh, fh);
                unpack8(wd, fd);
#pragma unroll
                for (int e = 0; e < 8; ++e) hsp += fh[e] * fd[e];
            }
            hsp += __shfl_xor(hsp, 16, 64);
            hsp += __shfl_xor(hsp, 32, 64);
            if (blk == 0 && g == 0) hs_s[ch] = hsp;
            const int jj = (t >> 1) - j0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * (t & 1) + i;
                const int c = 32 * (j0 + jj) + 8 * g + e;
                const float gg = G[jj][e] + (blk == 1 ? gend_s[0][c] : 0.f);  // chunk-global log2
                const float gam = exp2_hw(gg);
                const float gcr = exp2_hw(gend_s[0][c] + gend_s[1][c] - gg);  // Gam_C / Gam
                dqh[jj][e] += a.scale * gam * hq[i];
                const float dkg = -gam * hk[i];
                const float dkd = gcr * hd[i];
                dkh[jj][e] += dkg + dkd;
                dks[jj][e] += dkg - dkd;
                // sum over this block's tokens of k^ dk^_Kd for channel c
                const float kdr = row_sum16(kh[jj][e] * dkd);
                if (m == 0) kd_s[blk][c] = kdr;
            }
        }
    }
    // (no barrier: the next phase writes only tot_s and dot_s, which no wave
    // reads or writes in this one; the barrier after it publishes both phases)

    // ---- dG, its reverse cumulative sum over the chunk, and the chain rule
    float dla[KH][8];
#pragma unroll
    for (int jj = 0; jj < KH; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float dG = qh[jj][e] * dqh[jj][e] + kh[jj][e] * dks[jj][e];
            const float inc = row_scan16(dG);
            const float tot = __shfl(inc, (L & 48) | 15, 64);
            dla[jj][e] = tot - inc + dG;  // sum over this block's tokens s >= row
            if (blk == 1 && m == 15) tot_s[32 * (j0 + jj) + 8 * g + e] = tot;
        }
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int jj = 0; jj < KH; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) { pq += qh[jj][e] * dqh[jj][e]; pk += kh[jj][e] * dkh[jj][e]; }
    pq += __shfl_xor(pq, 16, 64);
    pq += __shfl_xor(pq, 32, 64);
    pk += __shfl_xor(pk, 16, 64);
    pk += __shfl_xor(pk, 32, 64);
    if (g == 0) { dot_s[hf][row][0] = pq; dot_s[hf][row][1] = pk; }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < KH; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 32 * (j0 + jj) + 8 * g + e;
            const float gc = exp2_hw(gend_s[0][c] + gend_s[1][c]);
            dla[jj][e] += (blk == 0 ? tot_s[c] : 0.f) + kd_s[0][c] + kd_s[1][c] + gc * hs_s[c];
        }

    // dq, dk through the norms
    pq = 0.f;
    pk = 0.f;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) { pq += dot_s[qq][row][0]; pk += dot_s[qq][row][1]; }
    if (valid) {
#pragma unroll
        for (int jj = 0; jj < KH; ++jj) {
            float xq[8], xk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xq[e] = (dqh[jj][e] - qh[jj][e] * pq) * iq;
                xk[e] = (dkh[jj][e] - kh[jj][e] * pk) * ik;
            }
            const int c0 = 32 * (j0 + jj) + 8 * g;
            *reinterpret_cast<bf16x8*>(a.dq + lrow * K + c0) = pack8(xq);
            *reinterpret_cast<bf16x8*>(a.dk + lrow * K + c0) = pack8(xk);
        }
    }
    // beta
    if (valid && hf == 0 && g == 0) {
        float db = 0.f;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) db += dbeta_s[qq][row];
        a.dbeta[lrow] = bits(GDN ? db : db * b * (1.f - b));
    }
    // the gate
    if constexpr (GDN) {
        float s = 0.f;
#pragma unroll
        for (int jj = 0; jj < KH; ++jj)
#pragma unroll
            for (int e = 0; e < 8; ++e) s += dla[jj][e];
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        __syncthreads();  // dot_s is reused
        if (g == 0) dot_s[hf][row][0] = s;
        __syncthreads();
        if (valid && hf == 0 && g == 0) {
            float d = 0.f;
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq) d += dot_s[qq][row][0];
            a.dg_gdn[lrow] = d;
        }
    } else {
        float alog = 0.f;
#pragma unroll
        for (int jj = 0; jj < KH; ++jj) {
            const int c0 = 32 * (j0 + jj) + 8 * g;
            float dx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xx = xg[jj][e];
                const float pre = -rate * softplus_f(xx);
                const float da = (valid && pre >= a.lower_bound) ? dla[jj][e] : 0.f;
                dx[e] = -rate * sigmoid_f(xx) * da;
                alog += da * pre;
                const float colsum = row_sum16(dx[e]);
                if (m == 0) red_s[blk][c0 + e] = colsum;
            }
            if (valid) *reinterpret_cast<bf16x8*>(a.dg_kda + lrow * K + c0) = pack8(dx);
        }
        alog += __shfl_xor(alog, 16, 64);
        alog += __shfl_xor(alog, 32, 64);
        alog = row_sum16(alog);
        if (L == 0) alog_s[wave] = alog;
        __syncthreads();
        for (int c = threadIdx.x; c < K; c += NT)
            a.part_dt[ch_base * K + c] = red_s[0][c] + red_s[1][c];
        if (threadIdx.x == 0) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < 2 * NQ; ++w) t += alog_s[w];
            a.part_alog[ch_base] = t;
        }
    }
}

template <int K, int V>
void launch_bwd_chunk_kv(const BwdArgs& a, bool gdn, int n_slots, hipStream_t stream) {
    const dim3 grid(n_slots * a.H), block(4 * K);
    if (gdn) hipLaunchKernelGGL((kda_bwd_chunk_kernel<K, V, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((kda_bwd_chunk_kernel<K, V, false>), grid, block, 0, stream, a);
}

void launch_bwd_chunk(const BwdArgs& a, int K, int V, bool gdn, int n_slots, hipStream_t stream) {
    if (n_slots <= 0) return;
    if (K == 128) {
        if (V == 128) launch_bwd_chunk_kv<128, 128>(a, gdn, n_slots, stream);
        else launch_bwd_chunk_kv<128, 64>(a, gdn, n_slots, stream);
    } else {
        if (V == 128) launch_bwd_chunk_kv<64, 128>(a, gdn, n_slots, stream);
        else launch_bwd_chunk_kv<64, 64>(a, gdn, n_slots, stream);
    }
}

// ------------------------------------------------------------ gate reductions
// dL/d(dt_bias)[h][c] and dL/dA_log[h]: sums over every chunk slot of the
// per-chunk sums, in a fixed order (no atomics: the result is reproducible).
// Workgroup (h, 64-channel block): thread (c, q) sums slots q, q + 4, ... of
// channel c; the four partial sums are added in LDS.  The workgroup with
// channel block 0 also sums dA_log's slots.
__global__ __launch_bounds__(256) void kda_bwd_reduce_kernel(const float* part_dt,
                                                             const float* part_alog,
                                                             int32_t n_slots, int32_t H,
                                                             int32_t K, float* ddt_bias,
                                                             float* dA_log) {
    __shared__ float acc[4][64];
    __shared__ float al[256];
    const int h = blockIdx.x, c = blockIdx.y * 64 + (threadIdx.x & 63), q = threadIdx.x >> 6;
    // eight independent partial sums, so eight loads are in flight at once;
    // the combination order is fixed, so the result is reproducible
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < K) {
        int sl = q;
        for (; sl + 28 < n_slots; sl += 32)
#pragma unroll
            for (int j = 0; j < 8; ++j) s[j] += part_dt[((int64_t)(sl + 4 * j) * H + h) * K + c];
#pragma unroll
        for (int j = 0; j < 7; ++j)
            if (sl + 4 * j < n_slots) s[j] += part_dt[((int64_t)(sl + 4 * j) * H + h) * K + c];
    }
    acc[q][threadIdx.x & 63] = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
    float t = 0.f;
    if (blockIdx.y == 0)
        for (int sl = threadIdx.x; sl < n_slots; sl += 256) t += part_alog[(int64_t)sl * H + h];
    al[threadIdx.x] = t;
    __syncthreads();
    if (q == 0 && c < K)
        ddt_bias[(int64_t)h * K + c] = (acc[0][threadIdx.x] + acc[1][threadIdx.x]) +
                                       (acc[2][threadIdx.x] + acc[3][threadIdx.x]);
    for (int d = 128; d > 0; d >>= 1) {
        if (threadIdx.x < d) al[threadIdx.x] += al[threadIdx.x + d];
        __syncthreads();
    }
    if (blockIdx.y == 0 && threadIdx.x == 0) dA_log[h] = al[0];
}

void launch_bwd_reduce(const float* part_dt, const float* part_alog, int32_t n_slots,
                       int32_t H, int32_t K, float* ddt_bias, float* dA_log, hipStream_t stream) {
    hipLaunchKernelGGL(kda_bwd_reduce_kernel, dim3(H, (K + 63) / 64), dim3(256), 0, stream,
                       part_dt, part_alog, n_slots, H, K, ddt_bias, dA_log);
}

}  // namespace kda
