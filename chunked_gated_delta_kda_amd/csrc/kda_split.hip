// kda_split.hip -- sequence splitting on one GPU (gfx950): the segment table
// and the scan that joins the segments.
//
// A long sequence has one chain of dependent chunk steps, so few long
// sequences leave most of the GPU idle.  Splitting each sequence into
// segments of L chunks makes the segments independent: with S_r the state
// entering segment r, the segment's effect is affine,
//   S_{r+1} = M_r S_r + N_r,
// where N_r is the segment's final state from a zero start and M_r (K x K)
// is the final "state" from an identity start with zero values (the product
// of the per-token transitions (I - b k k^T) Diag(a)).  One pass over all
// segments computes N_r and M_r, a short scan over segments gives every S_r,
// and a second pass recomputes each segment from its true S_r with outputs.
// This is the cross-rank algebra of context parallelism applied inside one
// card: the cuLA README (section "Benchmarks") reports FlashKDA's intra-card
// CP on long sequences, and the FlashQLA summary (section "핵심 기능")
// describes intra-card parallelism switched on when the gate's decay allows
// it.  Here M_r is computed only when the bound 2^(sum over the segment of
// max_c log2 a) on its norm is not negligible; otherwise S_{r+1} = N_r holds
// to far below fp32 rounding, so the shortcut stays exact.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int SEG_ORDER_BUCKETS = 1024;  // segment lengths (chunk steps) told apart
constexpr int SEG_WARM_CHUNKS = 1;       // the fused pass's first warm-up (kda_api.hip)

__device__ __forceinline__ int32_t block_scan_add(int32_t v, int32_t* buf) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int32_t o = tid >= d ? buf[tid - d] : 0;
        __syncthreads();
        buf[tid] += o;
        __syncthreads();
    }
    return buf[tid];  // inclusive
}

}  // namespace

// Virtual sequences = segments of at most L chunks of every sequence (an empty
// sequence keeps one empty segment, so its state passes through).  Inputs:
// the sequence table (seq_start, chunk_off over n_seqs).  Outputs, for
// n_virt_max virtual sequences: vseq_start / vchunk_off [n_virt_max + 1]
// (unused trailing entries are empty), final_map [n_virt_max] (the real
// sequence whose final state a last segment carries, else -1), vfirst
// [n_seqs + 1] (first virtual sequence of each real one).  The counts are
// bounded by construction: segments per sequence <= 1 + chunks / L, so
// their total never exceeds n_virt_max = n_seqs + ceil(slots / L).
__global__ __launch_bounds__(256) void kda_seg_table_kernel(const int32_t* seq_start,
                                                            const int32_t* chunk_off,
                                                            int32_t n_seqs, int32_t L,
                                                            int32_t n_virt_max,
                                                            int32_t* vseq_start,
                                                            int32_t* vchunk_off,
                                                            int32_t* final_map, int32_t* vfirst,
                                                            int32_t* order) {
    __shared__ int32_t buf[256];
    __shared__ int32_t hist[SEG_ORDER_BUCKETS];
    const int tid = threadIdx.x;
    int32_t carry = 0;
    for (int base = 0; base < n_seqs; base += 256) {
        const int n = base + tid;
        int32_t c0 = 0, c1 = 0, t0 = 0, t1 = 0, segs = 0;
        if (n < n_seqs) {
            c0 = chunk_off[n];
            c1 = chunk_off[n + 1];
            t0 = seq_start[n];
            t1 = seq_start[n + 1];
            segs = max(1, (c1 - c0 + L - 1) / L);
        }
        const int32_t incl = block_scan_add(segs, buf);
        const int32_t first = carry + incl - segs;
        if (n < n_seqs) {
            vfirst[n] = first;
            for (int r = 0; r < segs; ++r) {
                const int v = first + r;
                if (v >= n_virt_max) break;  // cannot happen (see the bound above)
                vchunk_off[v] = min(c0 + r * L, c1);
                vseq_start[v] = (int32_t)min((int64_t)t0 + (int64_t)r * L * C, (int64_t)t1);
                final_map[v] = r == segs - 1 ? n : -1;
            }
        }
        carry += buf[255];
        __syncthreads();
    }
    // the end of the last sequence closes every remaining (empty) entry
    const int32_t cend = n_seqs > 0 ? chunk_off[n_seqs] : 0;
    const int32_t tend = n_seqs > 0 ? seq_start[n_seqs] : 0;
    for (int v = carry + tid; v <= n_virt_max; v += 256) {
        vchunk_off[v] = cend;
        vseq_start[v] = tend;
        if (v < n_virt_max) final_map[v] = -1;
    }
    if (tid == 0) vfirst[n_seqs] = min(carry, n_virt_max);
    if (!order) return;

    // Dispatch order of the segments, longest first (list scheduling of
    // unequal jobs onto the compute units).  A segment's length in chunk
    // steps is its chunks plus the warm-up chunks of a segment that does not
    // start its sequence (the one after a sequence's last segment starts
    // one).  Counting sort on that length (clamped to the bucket count);
    // within a length the order is whatever the atomics give -- a segment's
    // results do not depend on when it runs.
    const int32_t nseg = min(carry, n_virt_max);
    __syncthreads();  // the table above is complete
    for (int i = tid; i < SEG_ORDER_BUCKETS; i += 256) hist[i] = 0;
    __syncthreads();
    auto bucket = [&](int v) {
        int32_t len = max(vchunk_off[v + 1] - vchunk_off[v], 0);
        if (v > 0 && final_map[v - 1] < 0) len += SEG_WARM_CHUNKS;
        return SEG_ORDER_BUCKETS - 1 - min(len, SEG_ORDER_BUCKETS - 1);
    };
    for (int v = tid; v < nseg; v += 256) atomicAdd(&hist[bucket(v)], 1);
    __syncthreads();
    constexpr int PER = SEG_ORDER_BUCKETS / 256;
    int32_t cnt[PER], sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        cnt[j] = hist[PER * tid + j];
        sum += cnt[j];
    }
    int32_t run = block_scan_add(sum, buf) - sum;  // exclusive prefix of this thread's buckets
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        hist[PER * tid + j] = run;
        run += cnt[j];
    }
    __syncthreads();
    for (int v = tid; v < nseg; v += 256) order[atomicAdd(&hist[bucket(v)], 1)] = v;
}

void launch_seg_table(const int32_t* seq_start, const int32_t* chunk_off, int32_t n_seqs,
                      int32_t L, int32_t n_virt_max, int32_t* vseq_start, int32_t* vchunk_off,
                      int32_t* final_map, int32_t* vfirst, hipStream_t stream, int32_t* order) {
    hipLaunchKernelGGL(kda_seg_table_kernel, dim3(1), dim3(256), 0, stream, seq_start, chunk_off,
                       n_seqs, L, n_virt_max, vseq_start, vchunk_off, final_map, vfirst, order);
}

// The scan over the segments of one (sequence, head, 32 value columns):
//   S = initial state;  for each segment r:  S_in[r] = S;  S = M_r S + N_r
// (M_r S dropped when its bound made it negligible).  S_in feeds the second
// pass.  Thread (rgp, col) holds rows 16 rgp .. 16 rgp + 15 of one column in
// fp32; M_r and S are staged in LDS for the product.
template <int K>
__global__ __launch_bounds__(256) void kda_split_scan_kernel(SplitScanArgs a) {
    constexpr int COLS = 32, RPT = K * COLS / 256;  // rows per thread (16 at K = 128)
    __shared__ float m_s[K][K + 1];
    __shared__ float s_s[K][COLS];
    const int VB = a.V / COLS;
    const int pair = blockIdx.x / VB, vb = blockIdx.x % VB;
    const int n = pair / a.H, h = pair % a.H;
    const int tid = threadIdx.x;
    const int col = tid % COLS, rgp = tid / COLS;
    const int c = vb * COLS + col;
    const int r0 = RPT * rgp;

    float S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        S[i] = a.initial_state
                   ? a.initial_state[(((int64_t)n * a.H + h) * K + r0 + i) * a.V + c]
                   : 0.f;
    const int v0 = a.vfirst[n], v1 = a.vfirst[n + 1];
    for (int v = v0; v < v1; ++v) {
        const int64_t base = ((int64_t)v * a.H + h) * K;
#pragma unroll
        for (int i = 0; i < RPT; ++i) a.s_in[(base + r0 + i) * a.V + c] = S[i];
        if (v == v1 - 1) break;  // the last segment's effect is the second pass's
        const bool full = a.trans_flag[(int64_t)v * a.H + h] != 0;  // uniform
        float nv[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) nv[i] = a.nstate[(base + r0 + i) * a.V + c];
        if (full) {
            __syncthreads();  // the previous step's LDS reads are done
            for (int e = tid; e < K * K; e += 256) m_s[e / K][e % K] = a.trans[base * K + e];
#pragma unroll
            for (int i = 0; i < RPT; ++i) s_s[r0 + i][col] = S[i];
            __syncthreads();
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                float acc = nv[i];
                for (int k = 0; k < K; ++k) acc += m_s[r0 + i][k] * s_s[k][col];
                S[i] = acc;
            }
        } else {
#pragma unroll
            for (int i = 0; i < RPT; ++i) S[i] = nv[i];
        }
    }
}

void launch_split_scan(const SplitScanArgs& a, int K, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.n_seqs * a.H * (a.V / 32);
    if (K == 128)
        hipLaunchKernelGGL(kda_split_scan_kernel<128>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(kda_split_scan_kernel<64>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, a);
}

}  // namespace kda
