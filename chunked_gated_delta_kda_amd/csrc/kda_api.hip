// kda_api.hip -- the C ABI of libkda (declared in include/kda.h): host-side
// argument checks, workspace layout and the launches (sequence table,
// kda_prep, kda_recur; the decode step) on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "kda.h"
#include "kda_common.h"
#include "kda_launch.h"

// Scratch of kda_fwd_noalloc: the packed-sequence and segment tables of the
// single-launch pass, in a device array of the library instead of a caller
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends; every call on that GPU shares it (the tables are rewritten
// in full by each call before they are read).
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t ALIGN = 256;
constexpr int VERSION = 100;  // 0.1.0

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool supported_dim(int32_t d) { return d == 64 || d == 128; }

// Chunk slots: an upper bound on sum over sequences of ceil(len / C).
int64_t max_slots(int32_t B, int32_t T, int32_t N, bool varlen) {
    if (!varlen) return (int64_t)B * ((T + kda::C - 1) / kda::C);
    return ((int64_t)B * T + kda::C - 1) / kda::C + N;
}

size_t meta_bytes(int32_t N) { return align_up(2 * sizeof(int32_t) * ((size_t)N + 1)); }

// Sequence splitting: segments of L chunks (L = 0: none).  n_virt bounds the
// number of segments (each sequence has at most 1 + chunks / L of them).
struct SplitPlan {
    int32_t L;
    int64_t n_virt;
};

constexpr int32_t SPLIT_MIN_CHUNKS = 64;      // shortest segment the automatic choice makes
constexpr int32_t SPLIT_MAX_BLOCKS = 128;     // it splits only below this many workgroups
constexpr int32_t SPLIT_TARGET_BLOCKS = 2048; // second-pass workgroups it aims for
constexpr int32_t RECUR_COLS = 32;         // value columns per kda_recur workgroup
constexpr float SPLIT_BOUND_LIMIT = -40.f; // log2: transitions below 2^-40 are negligible

// request: < 0 never split, 0 automatic, > 0 segment length in chunks.
SplitPlan plan_split(int32_t B, int32_t T, int32_t H, int32_t V, int32_t N, bool varlen,
                     int32_t request) {
    SplitPlan p{0, 0};
    const int64_t slots = max_slots(B, T, N, varlen);
    if (request < 0 || slots == 0) return p;
    int64_t L = request;
    if (request == 0) {
        // only when the (sequence, head, column block) workgroups leave most
        // CUs idle and the sequences are long
        const int64_t blocks = (int64_t)N * H * (V / RECUR_COLS);
        const int64_t avg = (slots + N - 1) / N;
        if (blocks >= SPLIT_MAX_BLOCKS || avg < 2 * SPLIT_MIN_CHUNKS) return p;
        const int64_t segs = (SPLIT_TARGET_BLOCKS + blocks - 1) / blocks;
        L = std::max<int64_t>(SPLIT_MIN_CHUNKS, (avg + segs - 1) / segs);
        if (L >= avg) return p;
    }
    p.L = (int32_t)std::min<int64_t>(L, INT32_MAX);
    p.n_virt = N + (slots + p.L - 1) / p.L;
    return p;
}

size_t bound_bytes(int64_t slots, int32_t H) { return align_up((size_t)slots * H * sizeof(float)); }

size_t split_bytes(const SplitPlan& p, int32_t N, int32_t H, int32_t K, int32_t V) {
    if (p.L == 0) return 0;
    const size_t nv = (size_t)p.n_virt;
    const size_t tables = align_up(sizeof(int32_t) * (2 * (nv + 1) + nv + ((size_t)N + 1)));
    const size_t flags = align_up(sizeof(int32_t) * nv * H);
    const size_t states = align_up(sizeof(float) * nv * H * K * V);
    const size_t trans = align_up(sizeof(float) * nv * H * K * K);
    return tables + flags + 2 * states + trans;
}

size_t workspace_bytes_for(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t N,
                           bool varlen, const SplitPlan& sp) {
    const int64_t slots = max_slots(B, T, N, varlen);
    return meta_bytes(N) + (size_t)slots * H * kda::record_bytes(K) + bound_bytes(slots, H) +
           split_bytes(sp, N, H, K, V);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Backward pass, after the forward layout (tables, records, bounds): the
// reverse-pass records, the chunk states and V - KG S of the forward sweep,
// the state gradients, dL/dU' and dL/dV of the reverse sweep (bf16), and the
// per-chunk sums of the gate-parameter gradients.
struct BwdLayout {
    unsigned char* brec;
    uint16_t *hs, *zt, *dss, *dut, *yt;
    float *part_dt, *part_alog;
};

size_t bwd_extra_bytes(int64_t slots, int32_t H, int32_t K, int32_t V) {
    const size_t ch = (size_t)slots * H;
    return align_up(ch * kda::record_bytes(K)) + 2 * align_up(ch * K * V * 2) +
           3 * align_up(ch * V * kda::C * 2) + align_up(ch * K * 4) + align_up(ch * 4);
}

BwdLayout bwd_layout(unsigned char* p, int64_t slots, int32_t H, int32_t K, int32_t V) {
    const size_t ch = (size_t)slots * H;
    BwdLayout b{};
    b.brec = p;
    p += align_up(ch * kda::record_bytes(K));
    b.hs = reinterpret_cast<uint16_t*>(p);
    p += align_up(ch * K * V * 2);
    b.dss = reinterpret_cast<uint16_t*>(p);
    p += align_up(ch * K * V * 2);
    b.zt = reinterpret_cast<uint16_t*>(p);
    p += align_up(ch * V * kda::C * 2);
    b.dut = reinterpret_cast<uint16_t*>(p);
    p += align_up(ch * V * kda::C * 2);
    b.yt = reinterpret_cast<uint16_t*>(p);
    p += align_up(ch * V * kda::C * 2);
    b.part_dt = reinterpret_cast<float*>(p);
    p += align_up(ch * K * 4);
    b.part_alog = reinterpret_cast<float*>(p);
    return b;
}

struct Common {
    const uint16_t *q, *k, *v, *beta;
    const float* initial_state;
    float* final_state;
    const int32_t* cu;  // read on the device by the prep stage only
    bool varlen;        // sequences packed along T (B == 1, N = num_seqs)
    int32_t num_seqs, B, T, H, K, V;
    uint16_t* o;
    void* ws;
    size_t ws_bytes;
    float scale;
    int32_t split;      // sequence-splitting request (see plan_split)
};

// Checks shared by both entry points; sets N.
// Token tensors may be NULL only when the batch holds no token (B * T == 0).
int check_common(const Common& c, int32_t& N) {
    if (c.B < 1 || c.T < 0 || c.H < 1) return KDA_ERR_INVALID_ARG;
    const bool tokens = c.T > 0;
    if (tokens && (!c.q || !c.k || !c.v || !c.beta || !c.o)) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(c.K) || !supported_dim(c.V)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)c.B * c.T >= ((int64_t)1 << 31)) return KDA_ERR_INVALID_ARG;
    if (!std::isfinite(c.scale)) return KDA_ERR_INVALID_ARG;
    if (c.varlen) {
        if (c.B != 1 || c.num_seqs < 1) return KDA_ERR_INVALID_ARG;
        N = c.num_seqs;
    } else {
        N = c.B;
    }
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.o, 8))
        return KDA_ERR_INVALID_ARG;
    if (!c.ws || !aligned(c.ws, ALIGN)) return KDA_ERR_WORKSPACE;
    const SplitPlan sp = plan_split(c.B, c.T, c.H, c.V, N, c.varlen, c.split);
    if (sp.n_virt > INT32_MAX / 4) return KDA_ERR_INVALID_ARG;
    if (c.ws_bytes < workspace_bytes_for(c.B, c.T, c.H, c.K, c.V, N, c.varlen, sp))
        return KDA_ERR_WORKSPACE;
    return KDA_OK;
}

struct WsLayout {
    int32_t* seq_start;
    int32_t* chunk_off;
    unsigned char* rec;
    float* bound;
    int64_t slots;
    SplitPlan sp;
    // splitting only
    int32_t *vseq_start, *vchunk_off, *final_map, *vfirst, *trans_flag;
    float *nstate, *trans, *s_in;
};

WsLayout layout(const Common& c, int32_t N) {
    WsLayout w{};
    unsigned char* base = static_cast<unsigned char*>(c.ws);
    w.seq_start = reinterpret_cast<int32_t*>(base);
    w.chunk_off = w.seq_start + (N + 1);
    w.slots = max_slots(c.B, c.T, N, c.varlen);
    size_t off = meta_bytes(N);
    w.rec = base + off;
    off += (size_t)w.slots * c.H * kda::record_bytes(c.K);
    w.bound = reinterpret_cast<float*>(base + off);
    off += bound_bytes(w.slots, c.H);
    w.sp = plan_split(c.B, c.T, c.H, c.V, N, c.varlen, c.split);
    if (w.sp.L > 0) {
        const size_t nv = (size_t)w.sp.n_virt;
        w.vseq_start = reinterpret_cast<int32_t*>(base + off);
        w.vchunk_off = w.vseq_start + (nv + 1);
        w.final_map = w.vchunk_off + (nv + 1);
        w.vfirst = w.final_map + nv;
        off += align_up(sizeof(int32_t) * (2 * (nv + 1) + nv + ((size_t)N + 1)));
        w.trans_flag = reinterpret_cast<int32_t*>(base + off);
        off += align_up(sizeof(int32_t) * nv * c.H);
        w.nstate = reinterpret_cast<float*>(base + off);
        off += align_up(sizeof(float) * nv * c.H * c.K * c.V);
        w.s_in = reinterpret_cast<float*>(base + off);
        off += align_up(sizeof(float) * nv * c.H * c.K * c.V);
        w.trans = reinterpret_cast<float*>(base + off);
    }
    return w;
}

// Sequence table and kda_prep: fills the workspace.
int run_prep(const Common& c, int32_t N, kda::PrepArgs p, bool gdn, hipStream_t stream,
             const kda::LaunchEvents* ev = nullptr) {
    const WsLayout w = layout(c, N);
    // (kda_prep's grid is one-dimensional over chunk slots x heads)
    if (w.slots * c.H > INT32_MAX || (int64_t)N * c.H * 2 > INT32_MAX) return KDA_ERR_INVALID_ARG;
    (void)hipGetLastError();  // clear a stale error from unrelated work
    if (c.varlen || w.sp.L > 0)  // splitting reads the table for fixed lengths too
        kda::launch_seq_table(c.varlen ? c.cu : nullptr, N, c.T, (int64_t)c.B * c.T,
                              w.seq_start, w.chunk_off, stream);
    p.q = c.q;
    p.k = c.k;
    p.beta = c.beta;
    p.H = c.H;
    p.n_seqs = N;
    p.packed = c.varlen;
    p.T = c.T;
    p.seq_start = w.seq_start;
    p.chunk_off = w.chunk_off;
    p.rec = w.rec;
    p.bound = w.bound;
    if (w.slots > 0) {
        kda::launch_prep(p, c.K, gdn, (int)w.slots, stream, ev);
    } else if (ev) {  // no kernel: the events still mark this point of the stream
        (void)hipEventRecord(ev->start, stream);
        (void)hipEventRecord(ev->stop, stream);
    }
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// kda_recur: consumes the workspace.  With splitting: the segment table, the
// first pass over all segments (results from a zero start and, where not
// negligible, transitions), the scan over segments and the second pass.
// ev (measurement events) applies to the unsplit recurrence only.
int run_recur(const Common& c, int32_t N, hipStream_t stream,
              const kda::LaunchEvents* ev = nullptr) {
    const WsLayout w = layout(c, N);
    if ((int64_t)N * c.H * 8 > INT32_MAX) return KDA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    kda::RecurArgs r{};
    r.v = c.v;
    r.rec = w.rec;
    r.initial_state = c.initial_state;
    r.final_state = c.final_state;
    r.o = c.o;
    r.scale = c.scale;
    r.H = c.H;
    r.V = c.V;
    r.n_seqs = N;
    r.packed = c.varlen;
    r.T = c.T;
    r.slot_limit = (int32_t)w.slots;
    r.tok_limit = (int64_t)c.B * c.T;
    r.seq_start = w.seq_start;
    r.chunk_off = w.chunk_off;
    if (w.sp.L == 0) {
        kda::launch_recur(r, c.K, stream, kda::RECUR_FWD, ev);
        return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
    }
    if (ev) return KDA_ERR_INVALID_ARG;
    const int32_t nv = (int32_t)w.sp.n_virt;
    if ((int64_t)nv * c.H * 8 > INT32_MAX) return KDA_ERR_INVALID_ARG;
    kda::launch_seg_table(w.seq_start, w.chunk_off, N, w.sp.L, nv, w.vseq_start, w.vchunk_off,
                          w.final_map, w.vfirst, stream);
    // first pass: every segment from a zero start, no outputs
    kda::RecurArgs p1 = r;
    p1.packed = 1;
    p1.n_seqs = nv;
    p1.seq_start = w.vseq_start;
    p1.chunk_off = w.vchunk_off;
    p1.initial_state = nullptr;
    p1.final_state = w.nstate;
    p1.o = nullptr;
    p1.trans_out = w.trans;
    p1.trans_flag = w.trans_flag;
    p1.bound = w.bound;
    p1.bound_limit = SPLIT_BOUND_LIMIT;
    p1.window = 1;  // a segment's zero-start end state needs only its decay window
    kda::launch_recur(p1, c.K, stream);
    kda::SplitScanArgs sa{};
    sa.initial_state = c.initial_state;
    sa.nstate = w.nstate;
    sa.trans = w.trans;
    sa.trans_flag = w.trans_flag;
    sa.vfirst = w.vfirst;
    sa.s_in = w.s_in;
    sa.H = c.H;
    sa.V = c.V;
    sa.n_seqs = N;
    kda::launch_split_scan(sa, c.K, stream);
    // second pass: every segment from its true entering state, with outputs
    kda::RecurArgs p2 = r;
    p2.packed = 1;
    p2.n_seqs = nv;
    p2.seq_start = w.vseq_start;
    p2.chunk_off = w.vchunk_off;
    p2.initial_state = w.s_in;
    p2.final_map = w.final_map;
    kda::launch_recur(p2, c.K, stream);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int run(const Common& c, int32_t N, kda::PrepArgs p, bool gdn, hipStream_t stream) {
    int st = run_prep(c, N, p, gdn, stream);
    return st != KDA_OK ? st : run_recur(c, N, stream);
}

// ---------------------------------------------- the single-launch forward pass
// One workgroup per (sequence segment, head) (kda_fused.hip).  Segments of L
// chunks: automatic (request 0) only when the (sequence, head) pairs are
// fewer than the compute units, aiming at one workgroup per unit, never
// shorter than FUSED_MIN_CHUNKS; a request < 0 keeps whole sequences, > 0
// sets L.  A segment that starts mid-sequence warms up over FUSED_WARM_CHUNKS
// chunks from a zero state, exact to 2^FUSED_BOUND_LIMIT of the entering
// state (fp32 rounding of the state), else over FUSED_WARM_RETRY chunks, else
// it restarts from the sequence start (see kda_fused.hip).  A failed attempt
// costs only its warm-up and pipeline-fill iterations.
constexpr int32_t FUSED_MIN_CHUNKS = 8;
constexpr int32_t FUSED_WARM_CHUNKS = 1;
constexpr int32_t FUSED_WARM_RETRY = 4;
// The plan targets MI355X's 256 compute units.  It is a constant, not a
// device query, so that the workspace size is a pure function of the sizes.
constexpr int64_t FUSED_CUS = 256;
constexpr float FUSED_BOUND_LIMIT = -24.f;

struct FusedPlan {
    int32_t L;             // chunks per segment
    int32_t segs_per_seq;  // fixed length
    int64_t n_virt;        // packed: segment slots (at most N + ceil(slots / L))
};

FusedPlan plan_fused(int32_t B, int32_t T, int32_t H, int32_t N, bool varlen, int32_t request) {
    FusedPlan p{1, 1, 0};
    const int64_t cus = FUSED_CUS;
    if (!varlen) {
        const int64_t nc = ((int64_t)T + kda::C - 1) / kda::C;
        int64_t L = std::max<int64_t>(nc, 1);
        if (request > 0) {
            L = request;
        } else if (request == 0) {
            const int64_t pairs = (int64_t)B * H;
            if (pairs < cus) {
                const int64_t segs = (cus + pairs - 1) / pairs;
                L = std::max<int64_t>(FUSED_MIN_CHUNKS, (nc + segs - 1) / segs);
            }
        }
        L = std::min<int64_t>(L, INT32_MAX);
        p.L = (int32_t)L;
        p.segs_per_seq = (int32_t)std::max<int64_t>(1, (nc + L - 1) / L);
    } else {
        const int64_t slots = ((int64_t)B * T + kda::C - 1) / kda::C + N;
        int64_t L = std::max<int64_t>(slots, 1);
        if (request > 0) {
            L = request;
        } else if (request == 0) {
            // about two workgroups per compute unit over the whole batch
            const int64_t work = slots * H;
            L = std::max<int64_t>(FUSED_MIN_CHUNKS, (work + 2 * cus - 1) / (2 * cus));
        }
        L = std::min<int64_t>(L, INT32_MAX);
        p.L = (int32_t)L;
        p.n_virt = N + (slots + L - 1) / L;
    }
    return p;
}

// Workspace of the single-launch pass: the packed-sequence and segment tables
// (nothing for fixed-length batches; one alignment unit is still reported,
// so that a size of 0 keeps meaning "unsupported").
size_t fused_workspace_bytes(const FusedPlan& p, int32_t N, bool varlen) {
    if (!varlen) return ALIGN;
    const size_t nv = (size_t)p.n_virt;
    return meta_bytes(N) + align_up(sizeof(int32_t) * (2 * (nv + 1) + nv + ((size_t)N + 1) + nv));
}

// Argument checks of the single-launch pass (its workspace instead of the
// two-stage one); sets N.
int check_fused(const Common& c, int32_t& N) {
    if (c.B < 1 || c.T < 0 || c.H < 1) return KDA_ERR_INVALID_ARG;
    const bool tokens = c.T > 0;
    if (tokens && (!c.q || !c.k || !c.v || !c.beta || !c.o)) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(c.K) || !supported_dim(c.V)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)c.B * c.T >= ((int64_t)1 << 31)) return KDA_ERR_INVALID_ARG;
    if (!std::isfinite(c.scale)) return KDA_ERR_INVALID_ARG;
    if (c.varlen) {
        if (c.B != 1 || c.num_seqs < 1) return KDA_ERR_INVALID_ARG;
        N = c.num_seqs;
    } else {
        N = c.B;
    }
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.o, 16) ||
        !aligned(c.beta, 2) || !aligned(c.initial_state, 16) || !aligned(c.final_state, 16))
        return KDA_ERR_INVALID_ARG;
    const FusedPlan fp = plan_fused(c.B, c.T, c.H, N, c.varlen, c.split);
    if (fp.n_virt > INT32_MAX / 4) return KDA_ERR_INVALID_ARG;
    const int64_t groups =
        c.varlen ? fp.n_virt * c.H : (int64_t)N * fp.segs_per_seq * c.H;
    if (groups > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (c.varlen) {
        if (!c.ws || !aligned(c.ws, ALIGN)) return KDA_ERR_WORKSPACE;
        if (c.ws_bytes < fused_workspace_bytes(fp, N, true)) return KDA_ERR_WORKSPACE;
    }
    return KDA_OK;
}

int run_fused(const Common& c, int32_t N, kda::FusedArgs f, bool gdn, hipStream_t stream,
              const kda::LaunchEvents* ev = nullptr) {
    const FusedPlan fp = plan_fused(c.B, c.T, c.H, N, c.varlen, c.split);
    (void)hipGetLastError();  // clear a stale error from unrelated work
    f.q = c.q;
    f.k = c.k;
    f.v = c.v;
    f.beta = c.beta;
    f.scale = c.scale;
    f.initial_state = c.initial_state;
    f.final_state = c.final_state;
    f.o = c.o;
    f.H = c.H;
    f.T = c.T;
    f.n_seqs = N;
    f.packed = c.varlen;
    f.warm_chunks = FUSED_WARM_CHUNKS;
    f.warm_chunks_retry = FUSED_WARM_RETRY;
    f.bound_limit = FUSED_BOUND_LIMIT;
    f.tok_limit = (int64_t)c.B * c.T;
    int64_t groups;
    if (!c.varlen) {
        f.seg_chunks = fp.L;
        f.segs_per_seq = fp.segs_per_seq;
        groups = (int64_t)N * fp.segs_per_seq * c.H;
    } else {
        const int32_t nv = (int32_t)fp.n_virt;
        unsigned char* base = static_cast<unsigned char*>(c.ws);
        int32_t* seq_start = reinterpret_cast<int32_t*>(base);
        int32_t* chunk_off = seq_start + (N + 1);
        int32_t* vseq_start = reinterpret_cast<int32_t*>(base + meta_bytes(N));
        int32_t* vchunk_off = vseq_start + (nv + 1);
        int32_t* final_map = vchunk_off + (nv + 1);
        int32_t* vfirst = final_map + nv;
        int32_t* order = vfirst + (N + 1);
        kda::launch_seq_table(c.cu, N, c.T, (int64_t)c.B * c.T, seq_start, chunk_off, stream);
        kda::launch_seg_table(seq_start, chunk_off, N, fp.L, nv, vseq_start, vchunk_off,
                              final_map, vfirst, stream, order);
        f.seq_start = seq_start;
        f.vseq_start = vseq_start;
        f.vfirst = vfirst;
        f.final_map = final_map;
        f.order = order;
        f.n_segs = nv;
        groups = (int64_t)nv * c.H;
    }
    kda::launch_fused(f, c.K, c.V, gdn, (int)groups, stream, ev);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

size_t fused_size_either_layout(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                int32_t num_seqs, int32_t segment_chunks) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 1 || !supported_dim(K) || !supported_dim(V))
        return 0;
    size_t need = 0;
    for (int varlen = 0; varlen < 2; ++varlen) {
        const int32_t N = varlen ? num_seqs : B;
        const FusedPlan fp = plan_fused(B, T, H, N, varlen != 0, segment_chunks);
        need = std::max(need, fused_workspace_bytes(fp, N, varlen != 0));
    }
    return need;
}

size_t bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t N,
                           bool varlen) {
    const SplitPlan none{0, 0};
    return align_up(workspace_bytes_for(B, T, H, K, V, N, varlen, none)) +
           bwd_extra_bytes(max_slots(B, T, N, varlen), H, K, V);
}

struct BwdIO {
    const uint16_t* d_o;
    const float* d_final;
    uint16_t *dq, *dk, *dv;
    uint16_t* dg_kda;
    float* dg_gdn;
    uint16_t* dbeta;
    float *dA_log, *ddt_bias, *dh0;
};

// The backward pass's share of its workspace (after the forward layout).
BwdLayout bwd_part(const Common& c, int32_t N, const WsLayout& w) {
    const SplitPlan none{0, 0};
    unsigned char* extra = static_cast<unsigned char*>(c.ws) +
                           align_up(workspace_bytes_for(c.B, c.T, c.H, c.K, c.V, N, c.varlen, none));
    return bwd_layout(extra, w.slots, c.H, c.K, c.V);
}

// kda_prep with the reverse-pass records, then the forward sweep that keeps
// every chunk's entering state and V - KG S: with outputs (a forward pass
// whose backward pass follows) or without (inside the backward pass).  KDA of
// fixed length with V = 128: the single-launch kernel's storing variant (it
// forms its own chunk operands in LDS, so the sweep reads only q, k, v, g and
// beta); otherwise the recurrence over the records (modes RECUR_FWD_STORE /
// RECUR_STORE).
int run_fwd_states(const Common& c, int32_t N, kda::PrepArgs p, bool gdn, bool outputs,
                   hipStream_t stream) {
    if (c.ws_bytes < bwd_workspace_bytes(c.B, c.T, c.H, c.K, c.V, N, c.varlen))
        return KDA_ERR_WORKSPACE;
    const WsLayout w = layout(c, N);
    if ((int64_t)N * c.H * 8 > INT32_MAX) return KDA_ERR_INVALID_ARG;  // recurrence grids
    const BwdLayout bl = bwd_part(c, N, w);
    p.brec = bl.brec;  // kda_prep also writes the reverse-pass records
    int st = run_prep(c, N, p, gdn, stream);
    if (st != KDA_OK) return st;
    Common cf = c;
    cf.split = 0;  // the single launch's own segment plan (the backward asks for none)
    if (!outputs) {
        cf.o = nullptr;
        cf.final_state = nullptr;
    }
    Common probe = cf;  // the single launch's own checks (alignment, grid size)
    if (!probe.o) probe.o = const_cast<uint16_t*>(probe.q);  // only checked, not written
    int32_t nf = 0;
    if (!c.varlen && !gdn && c.V == 128 && check_fused(probe, nf) == KDA_OK) {
        kda::FusedArgs f{};
        f.g_kda = p.g_kda;
        f.A_log = p.A_log;
        f.dt_bias = p.dt_bias;
        f.lower_bound = p.lower_bound;
        f.chunk_state = bl.hs;
        f.chunk_u = bl.zt;
        return run_fused(cf, N, f, gdn, stream);
    }
    (void)hipGetLastError();
    kda::RecurArgs r{};
    r.v = c.v;
    r.rec = w.rec;
    r.initial_state = c.initial_state;
    r.scale = c.scale;
    r.H = c.H;
    r.V = c.V;
    r.n_seqs = N;
    r.packed = c.varlen;
    r.T = c.T;
    r.slot_limit = (int32_t)w.slots;
    r.tok_limit = (int64_t)c.B * c.T;
    r.seq_start = w.seq_start;
    r.chunk_off = w.chunk_off;
    r.chunk_state = bl.hs;
    r.chunk_u = bl.zt;
    if (outputs) {
        r.o = c.o;
        r.final_state = c.final_state;
    }
    kda::launch_recur(r, c.K, stream, outputs ? kda::RECUR_FWD_STORE : kda::RECUR_STORE);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// The backward pass: the records and chunk states (recomputed, or left by a
// forward pass that saved them), the reverse sweep (state gradients, dv,
// dh0), the chunk gradient kernel and the gate-parameter sums.
int run_bwd(const Common& c, int32_t N, kda::PrepArgs p, bool gdn, const BwdIO& io,
            bool saved, hipStream_t stream) {
    if (c.ws_bytes < bwd_workspace_bytes(c.B, c.T, c.H, c.K, c.V, N, c.varlen))
        return KDA_ERR_WORKSPACE;
    const WsLayout w = layout(c, N);
    if ((int64_t)N * c.H * 8 > INT32_MAX) return KDA_ERR_INVALID_ARG;  // recurrence grids
    if (w.slots * c.H > INT32_MAX) return KDA_ERR_INVALID_ARG;  // chunk-gradient grid
    const BwdLayout bl = bwd_part(c, N, w);
    if (!saved) {
        const int st = run_fwd_states(c, N, p, gdn, false, stream);
        if (st != KDA_OK) return st;
    } else if (c.varlen) {
        // the sequence table indexes everything below: rebuilt from
        // cu_seqlens (clamped in range) rather than trusted from the workspace
        (void)hipGetLastError();
        kda::launch_seq_table(c.cu, N, c.T, (int64_t)c.B * c.T, w.seq_start, w.chunk_off, stream);
    }
    (void)hipGetLastError();
    kda::RecurArgs r{};
    r.v = c.v;
    r.rec = w.rec;
    r.initial_state = c.initial_state;
    r.scale = c.scale;
    r.H = c.H;
    r.V = c.V;
    r.n_seqs = N;
    r.packed = c.varlen;
    r.T = c.T;
    r.slot_limit = (int32_t)w.slots;
    r.tok_limit = (int64_t)c.B * c.T;
    r.seq_start = w.seq_start;
    r.chunk_off = w.chunk_off;
    r.chunk_state = bl.hs;
    r.chunk_u = bl.zt;
    kda::RecurArgs rb = r;
    rb.v = io.d_o;
    rb.rec = bl.brec;
    rb.initial_state = io.d_final;
    rb.final_state = io.dh0;
    rb.o = io.dv;
    rb.chunk_state = bl.dss;
    rb.chunk_u = bl.dut;
    rb.chunk_y = bl.yt;
    kda::launch_recur(rb, c.K, stream, kda::RECUR_BWD);
    kda::BwdArgs ba{};
    ba.q = c.q;
    ba.k = c.k;
    ba.g_kda = p.g_kda;
    ba.g_gdn = p.g_gdn;
    ba.beta = c.beta;
    ba.A_log = p.A_log;
    ba.dt_bias = p.dt_bias;
    ba.lower_bound = p.lower_bound;
    ba.scale = c.scale;
    ba.d_o = io.d_o;
    ba.dv = io.dv;
    ba.rec = w.rec;
    ba.hs = bl.hs;
    ba.zt = bl.zt;
    ba.dss = bl.dss;
    ba.dut = bl.dut;
    ba.yt = bl.yt;
    ba.dq = io.dq;
    ba.dk = io.dk;
    ba.dg_kda = io.dg_kda;
    ba.dg_gdn = io.dg_gdn;
    ba.dbeta = io.dbeta;
    ba.part_dt = bl.part_dt;
    ba.part_alog = bl.part_alog;
    ba.H = c.H;
    ba.n_seqs = N;
    ba.packed = c.varlen;
    ba.T = c.T;
    ba.seq_start = w.seq_start;
    ba.chunk_off = w.chunk_off;
    kda::launch_bwd_chunk(ba, c.K, c.V, gdn, (int)w.slots, stream);
    if (!gdn)
        kda::launch_bwd_reduce(bl.part_dt, bl.part_alog, (int32_t)w.slots, c.H, c.K, io.ddt_bias,
                               io.dA_log, stream);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// Pointer checks of the backward outputs (and the output gradient).
int check_bwd_io(const Common& c, const BwdIO& io, bool gdn) {
    const bool tokens = c.T > 0;
    if (tokens && (!io.d_o || !io.dq || !io.dk || !io.dv || !io.dbeta)) return KDA_ERR_INVALID_ARG;
    if (tokens && (gdn ? !io.dg_gdn : !io.dg_kda)) return KDA_ERR_INVALID_ARG;
    if (!gdn && (!io.dA_log || !io.ddt_bias)) return KDA_ERR_INVALID_ARG;
    if (!aligned(io.d_o, 16) || !aligned(io.dq, 16) || !aligned(io.dk, 16) ||
        !aligned(io.dv, 16) || !aligned(io.dg_kda, 16) || !aligned(io.dh0, 16) ||
        !aligned(io.d_final, 16))
        return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

// Checks of the KDA gate arguments.
int check_kda_gate(int32_t T, const uint16_t* g, const float* A_log, const float* dt_bias,
                   float lower_bound) {
    if ((T > 0 && !g) || !A_log || !dt_bias) return KDA_ERR_INVALID_ARG;
    if (!aligned(g, 16) || !aligned(dt_bias, 16)) return KDA_ERR_INVALID_ARG;
    if (!std::isfinite(lower_bound) || lower_bound < -5.f || lower_bound > 0.f)
        return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

// Checks shared by the decode entry points.
int check_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* beta,
                 float scale, const float* state_in, float* state_out, int32_t N, int32_t H,
                 int32_t K, int32_t V, const uint16_t* o) {
    if (N < 1 || H < 1) return KDA_ERR_INVALID_ARG;
    if (!q || !k || !v || !beta || !state_out || !o) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(K) || !supported_dim(V)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H * (V / 64) >= ((int64_t)1 << 31)) return KDA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 8) || !aligned(o, 8) ||
        !aligned(state_out, 16) || !aligned(state_in, 16))
        return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

int run_decode(kda::DecodeArgs& d, int32_t N, int32_t H, int32_t K, int32_t V, bool gdn,
               hipStream_t stream) {
    d.H = H;
    d.V = V;
    d.n_pairs = N * H;
    (void)hipGetLastError();
    kda::launch_decode(d, K, gdn, stream);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

namespace {

// Device address of `scratch` on each device, resolved once per device (the
// array's name in host code is only a stand-in for the symbol).
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return KDA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_fwd_split_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                    int32_t num_seqs, int32_t segment_chunks) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 1 || !supported_dim(K) || !supported_dim(V))
        return 0;
    // covers both layouts: packed sequences (num_seqs of them) and fixed length
    size_t need = 0;
    for (int varlen = 0; varlen < 2; ++varlen) {
        const SplitPlan sp = plan_split(B, T, H, V, num_seqs, varlen != 0, segment_chunks);
        need = std::max(need, workspace_bytes_for(B, T, H, K, V, num_seqs, varlen != 0, sp));
    }
    return need;
}

size_t kda_fwd_segmented_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                        int32_t num_seqs, int32_t segment_chunks) {
    return fused_size_either_layout(B, T, H, K, V, num_seqs, segment_chunks);
}

size_t kda_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t num_seqs) {
    return fused_size_either_layout(B, T, H, K, V, num_seqs, 0);
}

size_t gdn_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t num_seqs) {
    return fused_size_either_layout(B, T, H, K, V, num_seqs, 0);
}

int kda_fwd_split(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                  const uint16_t* beta, const float* A_log, const float* dt_bias,
                  float lower_bound, float scale, const float* initial_state,
                  float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                  int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                  size_t workspace_bytes, int32_t segment_chunks, void* stream) {
    Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, scale, segment_chunks};
    int st = check_kda_gate(T, g, A_log, dt_bias, lower_bound);
    if (st != KDA_OK) return st;
    int32_t N = 0;
    st = check_common(c, N);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_kda = g;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.lower_bound = lower_bound;
    return run(c, N, p, false, static_cast<hipStream_t>(stream));
}

static int kda_fwd_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* g, const uint16_t* beta, const float* A_log,
                         const float* dt_bias, float lower_bound, float scale,
                         const float* initial_state, float* final_state,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                         int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                         size_t workspace_bytes, int32_t segment_chunks, void* stream,
                         void* start_event, void* stop_event) {
    const bool timed = start_event || stop_event;
    if (timed && !(start_event && stop_event)) return KDA_ERR_INVALID_ARG;
    const kda::LaunchEvents ev{static_cast<hipEvent_t>(start_event),
                               static_cast<hipEvent_t>(stop_event)};
    Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, scale, segment_chunks};
    int st = check_kda_gate(T, g, A_log, dt_bias, lower_bound);
    if (st != KDA_OK) return st;
    int32_t N = 0;
    st = check_fused(c, N);
    if (st != KDA_OK) return st;
    kda::FusedArgs f{};
    f.g_kda = g;
    f.A_log = A_log;
    f.dt_bias = dt_bias;
    f.lower_bound = lower_bound;
    return run_fused(c, N, f, false, static_cast<hipStream_t>(stream), timed ? &ev : nullptr);
}

static int gdn_fwd_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                         const uint16_t* beta, float scale, const float* initial_state,
                         float* final_state, const int32_t* cu_seqlens, int32_t num_seqs,
                         int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o,
                         void* workspace, size_t workspace_bytes, int32_t segment_chunks,
                         void* stream, void* start_event, void* stop_event) {
    const bool timed = start_event || stop_event;
    if (timed && !(start_event && stop_event)) return KDA_ERR_INVALID_ARG;
    const kda::LaunchEvents ev{static_cast<hipEvent_t>(start_event),
                               static_cast<hipEvent_t>(stop_event)};
    Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, scale, segment_chunks};
    if (T > 0 && !g) return KDA_ERR_INVALID_ARG;
    int32_t N = 0;
    int st = check_fused(c, N);
    if (st != KDA_OK) return st;
    kda::FusedArgs f{};
    f.g_gdn = g;
    return run_fused(c, N, f, true, static_cast<hipStream_t>(stream), timed ? &ev : nullptr);
}

int kda_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
            const uint16_t* beta, const float* A_log, const float* dt_bias, float lower_bound,
            float scale, const float* initial_state, float* final_state,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
            int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
            void* stream) {
    return kda_fwd_fused(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
                         final_state, cu_seqlens, num_seqs, B, T, H, K, V, o, workspace,
                         workspace_bytes, 0, stream, nullptr, nullptr);
}

int kda_fwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                    const uint16_t* beta, const float* A_log, const float* dt_bias,
                    float lower_bound, float scale, const float* initial_state,
                    float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                    int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* stream) {
    // Every check of kda_fwd first, on the host, with the scratch standing
    // in as the workspace (a packed batch whose tables need more than the
    // array gets KDA_ERR_WORKSPACE); only then the array's device address.
    {
        Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
                 num_seqs, B, T, H, K, V, o, reinterpret_cast<void*>(ALIGN),
                 KDA_NOALLOC_SCRATCH_BYTES, scale, 0};
        int st = check_kda_gate(T, g, A_log, dt_bias, lower_bound);
        if (st != KDA_OK) return st;
        int32_t N = 0;
        st = check_fused(c, N);
        if (st != KDA_OK) return st;
    }
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (cu_seqlens != nullptr) {
        const int st = scratch_on_current_device(&ws);
        if (st != KDA_OK) return st;
        ws_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
    return kda_fwd_fused(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
                         final_state, cu_seqlens, num_seqs, B, T, H, K, V, o, ws, ws_bytes, 0,
                         stream, nullptr, nullptr);
}

int kda_fwd_segmented(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* g, const uint16_t* beta, const float* A_log,
                      const float* dt_bias, float lower_bound, float scale,
                      const float* initial_state, float* final_state, const int32_t* cu_seqlens,
                      int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                      uint16_t* o, void* workspace, size_t workspace_bytes,
                      int32_t segment_chunks, void* stream) {
    return kda_fwd_fused(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
                         final_state, cu_seqlens, num_seqs, B, T, H, K, V, o, workspace,
                         workspace_bytes, segment_chunks, stream, nullptr, nullptr);
}

int kda_fwd_timed(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                  const uint16_t* beta, const float* A_log, const float* dt_bias,
                  float lower_bound, float scale, const float* initial_state,
                  float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                  int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                  size_t workspace_bytes, void* stream, void* start_event, void* stop_event) {
    return kda_fwd_fused(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
                         final_state, cu_seqlens, num_seqs, B, T, H, K, V, o, workspace,
                         workspace_bytes, 0, stream, start_event, stop_event);
}

int gdn_fwd_split(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                  const uint16_t* beta, float scale, const float* initial_state,
                  float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                  int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                  size_t workspace_bytes, int32_t segment_chunks, void* stream) {
    Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, scale, segment_chunks};
    if (T > 0 && !g) return KDA_ERR_INVALID_ARG;
    int32_t N = 0;
    int st = check_common(c, N);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_gdn = g;
    return run(c, N, p, true, static_cast<hipStream_t>(stream));
}

int gdn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
            const uint16_t* beta, float scale, const float* initial_state, float* final_state,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
            int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
            void* stream) {
    return gdn_fwd_fused(q, k, v, g, beta, scale, initial_state, final_state, cu_seqlens,
                         num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, 0, stream,
                         nullptr, nullptr);
}

int gdn_fwd_segmented(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                      const uint16_t* beta, float scale, const float* initial_state,
                      float* final_state, const int32_t* cu_seqlens, int32_t num_seqs,
                      int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o,
                      void* workspace, size_t workspace_bytes, int32_t segment_chunks,
                      void* stream) {
    return gdn_fwd_fused(q, k, v, g, beta, scale, initial_state, final_state, cu_seqlens,
                         num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, segment_chunks,
                         stream, nullptr, nullptr);
}

int gdn_fwd_timed(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                  const uint16_t* beta, float scale, const float* initial_state,
                  float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                  int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                  size_t workspace_bytes, void* stream, void* start_event, void* stop_event) {
    return gdn_fwd_fused(q, k, v, g, beta, scale, initial_state, final_state, cu_seqlens,
                         num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, 0, stream,
                         start_event, stop_event);
}

int kda_prep_timed(const uint16_t* q, const uint16_t* k, const uint16_t* g,
                   const uint16_t* beta, const float* A_log, const float* dt_bias,
                   float lower_bound, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                   int32_t T, int32_t H, int32_t K, int32_t V, void* workspace,
                   size_t workspace_bytes, void* stream, void* start_event, void* stop_event) {
    const bool timed = start_event || stop_event;
    if (timed && !(start_event && stop_event)) return KDA_ERR_INVALID_ARG;
    const kda::LaunchEvents ev{static_cast<hipEvent_t>(start_event),
                               static_cast<hipEvent_t>(stop_event)};
    // v and o are not touched by this stage; stand-ins satisfy the shared checks
    Common c{q, k, q, beta, nullptr, nullptr, cu_seqlens, cu_seqlens != nullptr, num_seqs, B,
             T, H, K, V, const_cast<uint16_t*>(q), workspace, workspace_bytes, 1.f, -1};
    int st = check_kda_gate(T, g, A_log, dt_bias, lower_bound);
    if (st != KDA_OK) return st;
    int32_t N = 0;
    st = check_common(c, N);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_kda = g;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.lower_bound = lower_bound;
    return run_prep(c, N, p, false, static_cast<hipStream_t>(stream), timed ? &ev : nullptr);
}

int kda_prep(const uint16_t* q, const uint16_t* k, const uint16_t* g, const uint16_t* beta,
             const float* A_log, const float* dt_bias, float lower_bound,
             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
             int32_t K, int32_t V, void* workspace, size_t workspace_bytes, void* stream) {
    return kda_prep_timed(q, k, g, beta, A_log, dt_bias, lower_bound, cu_seqlens, num_seqs, B, T,
                          H, K, V, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int gdn_prep(const uint16_t* q, const uint16_t* k, const float* g, const uint16_t* beta,
             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
             int32_t K, int32_t V, void* workspace, size_t workspace_bytes, void* stream) {
    Common c{q, k, q, beta, nullptr, nullptr, cu_seqlens, cu_seqlens != nullptr, num_seqs, B,
             T, H, K, V, const_cast<uint16_t*>(q), workspace, workspace_bytes, 1.f, -1};
    if (T > 0 && !g) return KDA_ERR_INVALID_ARG;
    int32_t N = 0;
    int st = check_common(c, N);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_gdn = g;
    return run_prep(c, N, p, true, static_cast<hipStream_t>(stream));
}

int kda_recur_timed(const uint16_t* v, float scale, const float* initial_state,
                    float* final_state, int32_t varlen, int32_t num_seqs, int32_t B, int32_t T,
                    int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                    size_t workspace_bytes, void* stream, void* start_event, void* stop_event) {
    const bool timed = start_event || stop_event;
    if (timed && !(start_event && stop_event)) return KDA_ERR_INVALID_ARG;
    const kda::LaunchEvents ev{static_cast<hipEvent_t>(start_event),
                               static_cast<hipEvent_t>(stop_event)};
    // q, k, beta are not read by this stage; v stands in for them in the shared checks
    Common c{v, v, v, v, initial_state, final_state, nullptr, varlen != 0, num_seqs, B, T, H,
             K, V, o, workspace, workspace_bytes, scale, -1};
    int32_t N = 0;
    int st = check_common(c, N);
    if (st != KDA_OK) return st;
    return run_recur(c, N, static_cast<hipStream_t>(stream), timed ? &ev : nullptr);
}

int kda_recur(const uint16_t* v, float scale, const float* initial_state, float* final_state,
              int32_t varlen, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
              int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes, void* stream) {
    return kda_recur_timed(v, scale, initial_state, final_state, varlen, num_seqs, B, T, H, K, V,
                           o, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int kda_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
               const uint16_t* beta, const float* A_log, const float* dt_bias, float lower_bound,
               float scale, const float* state_in, float* state_out, int32_t N, int32_t H,
               int32_t K, int32_t V, uint16_t* o, void* stream) {
    int st = check_decode(q, k, v, beta, scale, state_in, state_out, N, H, K, V, o);
    if (st != KDA_OK) return st;
    st = check_kda_gate(1, g, A_log, dt_bias, lower_bound);
    if (st != KDA_OK) return st;
    kda::DecodeArgs d{};
    d.q = q;
    d.k = k;
    d.v = v;
    d.g_kda = g;
    d.beta = beta;
    d.A_log = A_log;
    d.dt_bias = dt_bias;
    d.lower_bound = lower_bound;
    d.scale = scale;
    d.state_in = state_in;
    d.state_out = state_out;
    d.o = o;
    return run_decode(d, N, H, K, V, false, static_cast<hipStream_t>(stream));
}

int gdn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
               const uint16_t* beta, float scale, const float* state_in, float* state_out,
               int32_t N, int32_t H, int32_t K, int32_t V, uint16_t* o, void* stream) {
    int st = check_decode(q, k, v, beta, scale, state_in, state_out, N, H, K, V, o);
    if (st != KDA_OK) return st;
    if (!g) return KDA_ERR_INVALID_ARG;
    kda::DecodeArgs d{};
    d.q = q;
    d.k = k;
    d.v = v;
    d.g_gdn = g;
    d.beta = beta;
    d.scale = scale;
    d.state_in = state_in;
    d.state_out = state_out;
    d.o = o;
    return run_decode(d, N, H, K, V, true, static_cast<hipStream_t>(stream));
}

size_t kda_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t num_seqs) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 1 || !supported_dim(K) || !supported_dim(V))
        return 0;
    return std::max(bwd_workspace_bytes(B, T, H, K, V, num_seqs, false),
                    bwd_workspace_bytes(B, T, H, K, V, num_seqs, true));
}

static int kda_bwd_run(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* g, const uint16_t* beta, const float* A_log,
                       const float* dt_bias, float lower_bound, float scale,
                       const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                       const uint16_t* d_o, const float* d_final, uint16_t* dq, uint16_t* dk,
                       uint16_t* dv, uint16_t* dg, uint16_t* dbeta, float* dA_log,
                       float* ddt_bias, float* dh0, void* workspace, size_t workspace_bytes,
                       void* stream, bool saved) {
    // dv stands in for the forward output in the shared checks
    Common c{q, k, v, beta, initial_state, nullptr, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, dv, workspace, workspace_bytes, scale, -1};
    const BwdIO io{d_o, d_final, dq, dk, dv, dg, nullptr, dbeta, dA_log, ddt_bias, dh0};
    int st = check_kda_gate(T, g, A_log, dt_bias, lower_bound);
    if (st != KDA_OK) return st;
    int32_t N = 0;
    st = check_common(c, N);
    if (st != KDA_OK) return st;
    st = check_bwd_io(c, io, false);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_kda = g;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.lower_bound = lower_bound;
    return run_bwd(c, N, p, false, io, saved, static_cast<hipStream_t>(stream));
}

int kda_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
            const uint16_t* beta, const float* A_log, const float* dt_bias, float lower_bound,
            float scale, const float* initial_state, const int32_t* cu_seqlens,
            int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
            const uint16_t* d_o, const float* d_final, uint16_t* dq, uint16_t* dk, uint16_t* dv,
            uint16_t* dg, uint16_t* dbeta, float* dA_log, float* ddt_bias, float* dh0,
            void* workspace, size_t workspace_bytes, void* stream) {
    return kda_bwd_run(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
                       cu_seqlens, num_seqs, B, T, H, K, V, d_o, d_final, dq, dk, dv, dg, dbeta,
                       dA_log, ddt_bias, dh0, workspace, workspace_bytes, stream, false);
}

int kda_bwd_saved(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                  const uint16_t* beta, const float* A_log, const float* dt_bias,
                  float lower_bound, float scale, const float* initial_state,
                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                  int32_t K, int32_t V, const uint16_t* d_o, const float* d_final, uint16_t* dq,
                  uint16_t* dk, uint16_t* dv, uint16_t* dg, uint16_t* dbeta, float* dA_log,
                  float* ddt_bias, float* dh0, void* workspace, size_t workspace_bytes,
                  void* stream) {
    return kda_bwd_run(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
                       cu_seqlens, num_seqs, B, T, H, K, V, d_o, d_final, dq, dk, dv, dg, dbeta,
                       dA_log, ddt_bias, dh0, workspace, workspace_bytes, stream, true);
}

static int gdn_bwd_run(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                       const uint16_t* beta, float scale, const float* initial_state,
                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                       int32_t H, int32_t K, int32_t V, const uint16_t* d_o,
                       const float* d_final, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                       float* dg, uint16_t* dbeta, float* dh0, void* workspace,
                       size_t workspace_bytes, void* stream, bool saved) {
    Common c{q, k, v, beta, initial_state, nullptr, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, dv, workspace, workspace_bytes, scale, -1};
    const BwdIO io{d_o, d_final, dq, dk, dv, nullptr, dg, dbeta, nullptr, nullptr, dh0};
    if (T > 0 && !g) return KDA_ERR_INVALID_ARG;
    int32_t N = 0;
    int st = check_common(c, N);
    if (st != KDA_OK) return st;
    st = check_bwd_io(c, io, true);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_gdn = g;
    return run_bwd(c, N, p, true, io, saved, static_cast<hipStream_t>(stream));
}

int gdn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
            const uint16_t* beta, float scale, const float* initial_state,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
            int32_t K, int32_t V, const uint16_t* d_o, const float* d_final, uint16_t* dq,
            uint16_t* dk, uint16_t* dv, float* dg, uint16_t* dbeta, float* dh0, void* workspace,
            size_t workspace_bytes, void* stream) {
    return gdn_bwd_run(q, k, v, g, beta, scale, initial_state, cu_seqlens, num_seqs, B, T, H, K,
                       V, d_o, d_final, dq, dk, dv, dg, dbeta, dh0, workspace, workspace_bytes,
                       stream, false);
}

int gdn_bwd_saved(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                  const uint16_t* beta, float scale, const float* initial_state,
                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                  int32_t K, int32_t V, const uint16_t* d_o, const float* d_final, uint16_t* dq,
                  uint16_t* dk, uint16_t* dv, float* dg, uint16_t* dbeta, float* dh0,
                  void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_bwd_run(q, k, v, g, beta, scale, initial_state, cu_seqlens, num_seqs, B, T, H, K,
                       V, d_o, d_final, dq, dk, dv, dg, dbeta, dh0, workspace, workspace_bytes,
                       stream, true);
}

int kda_fwd_save(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                 const uint16_t* beta, const float* A_log, const float* dt_bias,
                 float lower_bound, float scale, const float* initial_state, float* final_state,
                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                 int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
                 void* stream) {
    Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, scale, -1};
    int st = check_kda_gate(T, g, A_log, dt_bias, lower_bound);
    if (st != KDA_OK) return st;
    int32_t N = 0;
    st = check_common(c, N);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_kda = g;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.lower_bound = lower_bound;
    return run_fwd_states(c, N, p, false, true, static_cast<hipStream_t>(stream));
}

int gdn_fwd_save(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                 const uint16_t* beta, float scale, const float* initial_state, float* final_state,
                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                 int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
                 void* stream) {
    Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, scale, -1};
    if (T > 0 && !g) return KDA_ERR_INVALID_ARG;
    int32_t N = 0;
    int st = check_common(c, N);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_gdn = g;
    return run_fwd_states(c, N, p, true, true, static_cast<hipStream_t>(stream));
}

const char* kda_status_str(int status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG:
            return "invalid argument (null pointer, size, lower_bound, scale or alignment)";
        case KDA_ERR_UNSUPPORTED: return "unsupported head dimension (K and V must be 64 or 128)";
        case KDA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case KDA_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int kda_version(void) { return VERSION; }

}  // extern "C"
