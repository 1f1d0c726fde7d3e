// kda_api.hip -- the C ABI of libkda (declared in include/kda.h): host-side
// argument checks, workspace layout and the launches (sequence table,
// kda_prep, kda_recur; the decode step) on the caller's stream.
#include <cmath>
#include <cstdint>

#include "kda.h"
#include "kda_common.h"
#include "kda_launch.h"

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

size_t workspace_bytes_for(int32_t B, int32_t T, int32_t H, int32_t K, int32_t N, bool varlen) {
    return meta_bytes(N) + (size_t)max_slots(B, T, N, varlen) * H * kda::record_bytes(K);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

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
    if (c.ws_bytes < workspace_bytes_for(c.B, c.T, c.H, c.K, N, c.varlen))
        return KDA_ERR_WORKSPACE;
    return KDA_OK;
}

struct WsLayout {
    int32_t* seq_start;
    int32_t* chunk_off;
    unsigned char* rec;
    int64_t slots;
};

WsLayout layout(const Common& c, int32_t N) {
    WsLayout w;
    w.seq_start = static_cast<int32_t*>(c.ws);
    w.chunk_off = w.seq_start + (N + 1);
    w.rec = static_cast<unsigned char*>(c.ws) + meta_bytes(N);
    w.slots = max_slots(c.B, c.T, N, c.varlen);
    return w;
}

// Sequence table and kda_prep: fills the workspace.
int run_prep(const Common& c, int32_t N, kda::PrepArgs p, bool gdn, hipStream_t stream) {
    const WsLayout w = layout(c, N);
    if (w.slots > INT32_MAX || (int64_t)N * c.H * 2 > INT32_MAX) return KDA_ERR_INVALID_ARG;
    (void)hipGetLastError();  // clear a stale error from unrelated work
    if (c.varlen)
        kda::launch_seq_table(c.cu, N, c.T, (int64_t)c.B * c.T, w.seq_start, w.chunk_off,
                              stream);
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
    if (w.slots > 0) kda::launch_prep(p, c.K, gdn, (int)w.slots, stream);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// kda_recur: consumes the workspace.
int run_recur(const Common& c, int32_t N, hipStream_t stream) {
    const WsLayout w = layout(c, N);
    if ((int64_t)N * c.H * 2 > INT32_MAX) return KDA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    kda::RecurArgs r;
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
    r.seq_start = w.seq_start;
    r.chunk_off = w.chunk_off;
    kda::launch_recur(r, c.K, stream);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int run(const Common& c, int32_t N, kda::PrepArgs p, bool gdn, hipStream_t stream) {
    int st = run_prep(c, N, p, gdn, stream);
    return st != KDA_OK ? st : run_recur(c, N, stream);
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

extern "C" {

size_t kda_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t num_seqs) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 1 || !supported_dim(K) || !supported_dim(V))
        return 0;
    // the bound for packed sequences also covers the fixed-length layout (N = B)
    return workspace_bytes_for(B, T, H, K, num_seqs, true);
}

size_t gdn_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t num_seqs) {
    return kda_fwd_workspace_size(B, T, H, K, V, num_seqs);
}

int kda_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
            const uint16_t* beta, const float* A_log, const float* dt_bias, float lower_bound,
            float scale, const float* initial_state, float* final_state,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
            int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
            void* stream) {
    Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, scale};
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

int gdn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
            const uint16_t* beta, float scale, const float* initial_state, float* final_state,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
            int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
            void* stream) {
    Common c{q, k, v, beta, initial_state, final_state, cu_seqlens, cu_seqlens != nullptr,
             num_seqs, B, T, H, K, V, o, workspace, workspace_bytes, scale};
    if (T > 0 && !g) return KDA_ERR_INVALID_ARG;
    int32_t N = 0;
    int st = check_common(c, N);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_gdn = g;
    return run(c, N, p, true, static_cast<hipStream_t>(stream));
}

int kda_prep(const uint16_t* q, const uint16_t* k, const uint16_t* g, const uint16_t* beta,
             const float* A_log, const float* dt_bias, float lower_bound,
             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
             int32_t K, int32_t V, void* workspace, size_t workspace_bytes, void* stream) {
    // v and o are not touched by this stage; stand-ins satisfy the shared checks
    Common c{q, k, q, beta, nullptr, nullptr, cu_seqlens, cu_seqlens != nullptr, num_seqs, B,
             T, H, K, V, const_cast<uint16_t*>(q), workspace, workspace_bytes, 1.f};
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
    return run_prep(c, N, p, false, static_cast<hipStream_t>(stream));
}

int gdn_prep(const uint16_t* q, const uint16_t* k, const float* g, const uint16_t* beta,
             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
             int32_t K, int32_t V, void* workspace, size_t workspace_bytes, void* stream) {
    Common c{q, k, q, beta, nullptr, nullptr, cu_seqlens, cu_seqlens != nullptr, num_seqs, B,
             T, H, K, V, const_cast<uint16_t*>(q), workspace, workspace_bytes, 1.f};
    if (T > 0 && !g) return KDA_ERR_INVALID_ARG;
    int32_t N = 0;
    int st = check_common(c, N);
    if (st != KDA_OK) return st;
    kda::PrepArgs p{};
    p.g_gdn = g;
    return run_prep(c, N, p, true, static_cast<hipStream_t>(stream));
}

int kda_recur(const uint16_t* v, float scale, const float* initial_state, float* final_state,
              int32_t varlen, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
              int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes, void* stream) {
    // q, k, beta are not read by this stage; v stands in for them in the shared checks
    Common c{v, v, v, v, initial_state, final_state, nullptr, varlen != 0, num_seqs, B, T, H,
             K, V, o, workspace, workspace_bytes, scale};
    int32_t N = 0;
    int st = check_common(c, N);
    if (st != KDA_OK) return st;
    return run_recur(c, N, static_cast<hipStream_t>(stream));
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
