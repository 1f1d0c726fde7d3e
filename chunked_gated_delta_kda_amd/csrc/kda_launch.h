// kda_launch.h -- host-side launch interface between the C-ABI layer and the
// two kernels.  Pointers are device pointers; bf16 tensors are passed as
// uint16_t bit patterns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct PrepArgs {
    const uint16_t* q;         // [tokens, H, K] bf16
    const uint16_t* k;         // [tokens, H, K] bf16
    const uint16_t* g_kda;     // KDA: pre-activation gate [tokens, H, K] bf16
    const float* g_gdn;        // GDN: log decay [tokens, H] fp32
    const uint16_t* beta;      // [tokens, H] bf16 (KDA logits / GDN probabilities)
    const float* A_log;        // [H] (KDA)
    const float* dt_bias;      // [H, K] (KDA)
    float lower_bound;         // KDA floor of the log decay
    int32_t H;
    int32_t n_seqs;
    int32_t packed;            // 0: fixed length (every sequence has T tokens)
    int32_t T;                 // tokens per sequence when not packed
    const int32_t* seq_start;  // packed: [n_seqs + 1] flattened token offsets
    const int32_t* chunk_off;  // packed: [n_seqs + 1] first chunk slot of each sequence
    unsigned char* rec;        // [slots, H, record bytes]
    float* bound;              // [slots, H]: sum over the chunk of max_c log2 a (<= 0)
    unsigned char* brec;       // [slots, H, BRec bytes] or null: the reverse-pass records
};

struct RecurArgs {
    const uint16_t* v;             // [tokens, H, V] bf16
    const unsigned char* rec;      // records from kda_prep
    const float* initial_state;    // [n_seqs, H, K, V] or null (zeros)
    float* final_state;            // [n_seqs, H, K, V] or null (not written)
    uint16_t* o;                   // [tokens, H, V] bf16
    float scale;
    int32_t H;
    int32_t V;
    int32_t n_seqs;
    int32_t packed;
    int32_t T;
    const int32_t* seq_start;
    const int32_t* chunk_off;
    // Bounds known on the host: chunk slots in the workspace and tokens in the
    // batch.  Every range read from seq_start / chunk_off is clamped to them,
    // so a table that does not match these arguments (a workspace filled for
    // other sizes, or never filled) cannot send an access out of bounds.
    int32_t slot_limit;
    int64_t tok_limit;
    // Sequence splitting (all null / 0 for the plain forward pass):
    const int32_t* final_map;  // [n_seqs] or null: final state of sequence n goes to
                               // final_state[final_map[n]] (skipped when < 0)
    float* trans_out;          // [n_seqs, H, K, K] or null: also run K transition
                               // columns (identity start, zero values) and store them
    int32_t* trans_flag;       // [n_seqs, H]: 1 when trans_out was computed, 0 when the
                               // bound showed the transition negligible (not computed)
    const float* bound;        // [slots, H] chunk bounds from kda_prep (log2)
    float bound_limit;         // a transition with a summed bound below this is negligible
    int32_t window;            // 1: value columns start at the segment's decay window
    // Backward pass (null for the forward pass):
    uint16_t* chunk_state;     // [slots, H, K, V] bf16: the state entering each chunk
                               // (reverse pass: the state gradient leaving each chunk)
    uint16_t* chunk_u;         // [slots, H, V, C] bf16, tokens in k-slot order: the
                               // chunk's V - KG S (reverse pass: dL/dU')
    uint16_t* chunk_y;         // reverse pass: [slots, H, V, C] bf16, dL/dV in the same
                               // layout (or null)
};

// kda_recur variants: the forward pass; the forward pass that stores every
// chunk's entering state and V - KG S instead of outputs; the reverse pass
// over the backward record (state gradient, dL/dU' and dv); the forward pass
// with its outputs that also stores what the state-store variant stores.
enum RecurMode { RECUR_FWD = 0, RECUR_STORE = 1, RECUR_BWD = 2, RECUR_FWD_STORE = 3 };

struct DecodeArgs {
    const uint16_t* q;         // [pairs, K] bf16 (pairs = N * H, head fastest)
    const uint16_t* k;         // [pairs, K] bf16
    const uint16_t* v;         // [pairs, V] bf16
    const uint16_t* g_kda;     // KDA: pre-activation gate [pairs, K] bf16
    const float* g_gdn;        // GDN: log decay [pairs] fp32
    const uint16_t* beta;      // [pairs] bf16 (KDA logits / GDN probabilities)
    const float* A_log;        // [H] (KDA)
    const float* dt_bias;      // [H, K] (KDA)
    float lower_bound;
    float scale;
    const float* state_in;     // [pairs, K, V] fp32 or null (zeros)
    float* state_out;          // [pairs, K, V] fp32 (may equal state_in)
    uint16_t* o;               // [pairs, V] bf16
    int32_t H;
    int32_t V;
    int32_t n_pairs;
};

struct SplitScanArgs {
    const float* initial_state;  // [n_seqs, H, K, V] or null (zeros)
    const float* nstate;         // [virtual, H, K, V]: segment results from a zero start
    const float* trans;          // [virtual, H, K, K]: segment transitions
    const int32_t* trans_flag;   // [virtual, H]: transition computed (else negligible)
    const int32_t* vfirst;       // [n_seqs + 1]: first segment of each sequence
    float* s_in;                 // [virtual, H, K, V]: state entering each segment
    int32_t H;
    int32_t V;
    int32_t n_seqs;
};

// The single-launch forward pass (kda_fused.hip): one workgroup per
// (sequence segment, head).  Fixed-length batches: sequence n is tokens
// [n T, (n+1) T), cut into segs_per_seq segments of seg_chunks chunks.
// Packed batches: the segment table of kda_seg_table (vseq_start, vfirst,
// final_map over n_segs segment slots) and the sequence table (seq_start).
struct FusedArgs {
    const uint16_t* q;          // [tokens, H, K] bf16
    const uint16_t* k;          // [tokens, H, K] bf16
    const uint16_t* v;          // [tokens, H, V] bf16
    const uint16_t* g_kda;      // KDA: pre-activation gate [tokens, H, K] bf16
    const float* g_gdn;         // GDN: log decay [tokens, H] fp32
    const uint16_t* beta;       // [tokens, H] bf16 (KDA logits / GDN probabilities)
    const float* A_log;         // [H] (KDA)
    const float* dt_bias;       // [H, K] (KDA)
    float lower_bound;
    float scale;
    const float* initial_state; // [n_seqs, H, K, V] or null (zeros)
    float* final_state;         // [n_seqs, H, K, V] or null (not written)
    uint16_t* o;                // [tokens, H, V] bf16
    int32_t H;
    int32_t T;                  // tokens per sequence (fixed length)
    int32_t n_seqs;
    int32_t packed;
    int32_t seg_chunks;         // fixed length: chunks per segment
    int32_t segs_per_seq;       // fixed length: segments per sequence
    int32_t n_segs;             // packed: segment slots in the tables
    const int32_t* seq_start;   // packed: [n_seqs + 1] token offsets
    const int32_t* vseq_start;  // packed: [n_segs + 1] first token of each segment
    const int32_t* vfirst;      // packed: [n_seqs + 1] first segment of each sequence
    const int32_t* final_map;   // packed: [n_segs] sequence whose final state a segment ends
    const int32_t* order;       // packed: [n_segs] segment of each dispatch rank (or null)
    int32_t warm_chunks;        // warm-up chunks before a segment that starts mid-sequence
    int32_t warm_chunks_retry;  // the second attempt's warm-up (after a failed bound)
    float bound_limit;          // log2: a warm-up whose transitions are below this suffices
    int64_t tok_limit;          // tokens in the batch
    // KDA of fixed length with V = 128 only (null otherwise): with chunk_state
    // set, every chunk's entering state and V - KG S are stored, in the layouts
    // of RecurArgs' fields of the same names, and o may be null (no outputs)
    uint16_t* chunk_state;      // [slots, H, K, V] bf16
    uint16_t* chunk_u;          // [slots, H, V, C] bf16, tokens in k-slot order
};

// Backward pass: the chunk-parallel gradient kernel (kda_bwd.hip).
struct BwdArgs {
    const uint16_t* q;         // [tokens, H, K] bf16
    const uint16_t* k;         // [tokens, H, K] bf16
    const uint16_t* g_kda;     // KDA: pre-activation gate [tokens, H, K] bf16
    const float* g_gdn;        // GDN: log decay [tokens, H] fp32
    const uint16_t* beta;      // [tokens, H] bf16
    const float* A_log;        // [H] (KDA)
    const float* dt_bias;      // [H, K] (KDA)
    float lower_bound;
    float scale;
    const uint16_t* d_o;       // [tokens, H, V] bf16: dL/do
    const uint16_t* dv;        // [tokens, H, V] bf16: dL/dv (from the reverse pass)
    const unsigned char* rec;  // forward records (for Tb)
    const uint16_t* hs;        // [slots, H, K, V] bf16: state entering each chunk
    const uint16_t* zt;        // [slots, H, V, C] bf16: V - KG S of each chunk
    const uint16_t* dss;       // [slots, H, K, V] bf16: gradient of the state leaving it
    const uint16_t* dut;       // [slots, H, V, C] bf16: dL/dU'
    const uint16_t* yt;        // [slots, H, V, C] bf16: dL/dV (token-ordered copy of dv)
    uint16_t* dq;              // [tokens, H, K] bf16
    uint16_t* dk;              // [tokens, H, K] bf16
    uint16_t* dg_kda;          // KDA: [tokens, H, K] bf16
    float* dg_gdn;             // GDN: [tokens, H] fp32
    uint16_t* dbeta;           // [tokens, H] bf16
    float* part_dt;            // KDA: [slots, H, K] per-chunk sums of dL/d(dt_bias)
    float* part_alog;          // KDA: [slots, H] per-chunk sums of dL/dA_log
    int32_t H;
    int32_t n_seqs;
    int32_t packed;
    int32_t T;
    const int32_t* seq_start;
    const int32_t* chunk_off;
};

void launch_bwd_chunk(const BwdArgs& a, int K, int V, bool gdn, int n_slots, hipStream_t stream);
void launch_bwd_reduce(const float* part_dt, const float* part_alog, int32_t n_slots,
                       int32_t H, int32_t K, float* ddt_bias, float* dA_log, hipStream_t stream);

// order (optional, [n_virt_max]): the segments longest first, for dispatch
void launch_seg_table(const int32_t* seq_start, const int32_t* chunk_off, int32_t n_seqs,
                      int32_t L, int32_t n_virt_max, int32_t* vseq_start, int32_t* vchunk_off,
                      int32_t* final_map, int32_t* vfirst, hipStream_t stream,
                      int32_t* order = nullptr);
void launch_split_scan(const SplitScanArgs& a, int K, hipStream_t stream);
void launch_seq_table(const int32_t* cu, int32_t n_seqs, int32_t T, int64_t total_tokens,
                      int32_t* seq_start, int32_t* chunk_off, hipStream_t stream);
// Measurement events for a stage's main kernel (both non-null or ev null):
// the kernel is then launched with hipExtLaunchKernel, which records its own
// start and end on the GPU into the two events.
struct LaunchEvents {
    hipEvent_t start;
    hipEvent_t stop;
};

void launch_prep(const PrepArgs& a, int K, bool gdn, int n_slots, hipStream_t stream,
                 const LaunchEvents* ev = nullptr);
void launch_recur(const RecurArgs& a, int K, hipStream_t stream, RecurMode mode = RECUR_FWD,
                  const LaunchEvents* ev = nullptr);
void launch_decode(const DecodeArgs& a, int K, bool gdn, hipStream_t stream);
void launch_fused(const FusedArgs& a, int K, int V, bool gdn, int n_groups, hipStream_t stream,
                  const LaunchEvents* ev = nullptr);
int record_bytes(int K);
// compute units of the current device (queried once per device)
int device_cus();

}  // namespace kda
