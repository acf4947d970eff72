// kda_api.hip -- the extern "C" boundary of libkda: argument validation,
// workspace sizing and kernel launches.  See include/kda.h for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/kda.h"

#include "kda_internal.h"

namespace {

constexpr int CHUNK = 64;
// Record budget of one window: records written by the chunk-local pass should
// still sit in the 256 MB last-level (MALL) cache when the state pass reads
// them.  The chunk-local pass streams its inputs and outputs with non-temporal
// accesses, so records of up to about 230 MB stay resident; past that the state
// pass starts missing.
constexpr size_t RECORD_BUDGET = size_t(220) << 20;
constexpr int64_t MIN_WINDOW = 32;
constexpr size_t WINDOW_CAP = size_t(4) << 30;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

// A C caller may store any int in an enum field or pass any int for an enum
// parameter; in C++ a value outside the enumerators' range may not be read as the
// enum type, so the library reads every caller-supplied enum's bits as an int.
template <typename E>
int enum_code(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "the ABI's enums are ints");
    int x;
    memcpy(&x, &e, sizeof(x));
    return x;
}

size_t dsize(int t) { return t == KDA_DTYPE_BF16 ? 2 : 4; }

struct Range {
    const void* p;
    size_t n;
};

// True when [x, x + xn) overlaps any of the ranges (null or empty ranges never do).
template <size_t K>
bool overlaps_any(const void* x, size_t xn, const Range (&rs)[K]) {
    for (const Range& r : rs)
        if (overlaps(x, xn, r.p, r.n)) return true;
    return false;
}

struct Plan {
    int64_t N, tokens, max_len, max_chunks;
    int d;
    size_t rec, state_bytes;
};

kda_status_t plan_chunk(const kda_shape_t* s, Plan& p) {
    if (!s) return KDA_ERR_INVALID_ARG;
    if (s->heads <= 0 || s->batch <= 0 || s->seqlen < 0 || s->dk <= 0 || s->dv <= 0 || s->max_seqlen < 0)
        return KDA_ERR_INVALID_ARG;
    const int in_t = enum_code(s->in_dtype), out_t = enum_code(s->out_dtype);
    if ((in_t != KDA_DTYPE_F32 && in_t != KDA_DTYPE_BF16) || (out_t != KDA_DTYPE_F32 && out_t != KDA_DTYPE_BF16))
        return KDA_ERR_UNSUPPORTED;
    if (s->dk != s->dv || (s->dk != 64 && s->dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (s->gate_per_head != 0 && s->gate_per_head != 1) return KDA_ERR_INVALID_ARG;
    p.d = s->dk;
    return KDA_OK;
}

// Scratch of kda_chunk_fwd_noalloc: one array per device the library runs on,
// held until the process ends.  Host code must never pass `scratch` itself to a
// kernel (in host code the name is a stand-in, not a device address): the device
// address is looked up once per device and kept in g_scratch.
constexpr size_t NOALLOC_SCRATCH_BYTES = KDA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::once_flag g_scratch_once[MAX_DEVICES];
void* g_scratch[MAX_DEVICES];
hipError_t g_scratch_err[MAX_DEVICES];

// The current device's scratch address (null if the device index is out of range
// or the lookup failed).
void* device_scratch(hipError_t& err) {
    int dev = -1;
    err = hipGetDevice(&dev);
    if (err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= MAX_DEVICES) {
        err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    err = g_scratch_err[dev];
    return g_scratch[dev];
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status_t st) {
    // A C caller may pass any int; in C++ a value outside the enumerators' range may not
    // be read as kda_status_t, so the argument's bits are read as an int.
    int code;
    static_assert(sizeof(code) == sizeof(st), "kda_status_t is an int");
    memcpy(&code, &st, sizeof(code));
    switch (code) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

// KDA_CHECK=1: copy cu_seqlens to the host (synchronising `stream`) and verify
// the preconditions the kernels rely on: cu[0] = 0, non-decreasing, cu[N] =
// total tokens, no sequence longer than the max_seqlen the launch is sized for.
static kda_status_t check_cu_seqlens(const int32_t* cu, const Plan& p, hipStream_t stream) {
    std::vector<int32_t> h((size_t)p.N + 1);
    if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return KDA_ERR_HIP;
    if (h[0] != 0 || h[(size_t)p.N] != p.tokens) return KDA_ERR_INVALID_ARG;
    for (int64_t i = 0; i < p.N; ++i) {
        const int64_t len = (int64_t)h[(size_t)i + 1] - h[(size_t)i];
        if (len < 0 || len > p.max_len) return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

// Under KDA_CHECK=1 with bf16 inputs: the largest |v| and |initial state|,
// measured on the device (synchronising `stream`).  Past F16_RANGE_SAFE the
// call runs with fp32 matrix-core operands and records instead of fp16 ones,
// whose range (6.5e4) values a few times larger would leave.  `scratch` is
// 2 * RANGE_BLOCKS floats of the workspace, written before any kernel of the
// call uses it.
constexpr float F16_RANGE_SAFE = 1024.f;
constexpr int RANGE_BLOCKS = 256;

static kda_status_t needs_f32_operands(const void* v, size_t nv, const float* init, size_t ninit, float* scratch,
                                       hipStream_t stream, bool& f32) {
    f32 = false;
    if (nv == 0 && ninit == 0) return KDA_OK;
    if (nv && kda::max_abs_dispatch(v, nv, true, scratch, RANGE_BLOCKS, stream) != hipSuccess) return KDA_ERR_HIP;
    if (ninit && kda::max_abs_dispatch(init, ninit, false, scratch + RANGE_BLOCKS, RANGE_BLOCKS, stream) != hipSuccess)
        return KDA_ERR_HIP;
    std::vector<float> h(2 * RANGE_BLOCKS, 0.f);
    if (nv && hipMemcpyAsync(h.data(), scratch, RANGE_BLOCKS * sizeof(float), hipMemcpyDeviceToHost, stream) !=
                  hipSuccess)
        return KDA_ERR_HIP;
    if (ninit && hipMemcpyAsync(h.data() + RANGE_BLOCKS, scratch + RANGE_BLOCKS, RANGE_BLOCKS * sizeof(float),
                                hipMemcpyDeviceToHost, stream) != hipSuccess)
        return KDA_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return KDA_ERR_HIP;
    float m = 0.f;
    for (float x : h) m = x > m ? x : m;  // a NaN block maximum is +inf
    f32 = !(m <= F16_RANGE_SAFE);
    return KDA_OK;
}

static bool check_enabled() {
    const char* chk = getenv("KDA_CHECK");
    return chk && chk[0] == '1';
}

// Bytes of one per-segment state array [units, G, d, d] fp32 (256-aligned).
static size_t segment_bytes(const Plan& p, int heads, int G) {
    return align256((size_t)p.N * heads * G * p.d * p.d * sizeof(float));
}

static kda_status_t chunk_plan_full(const kda_shape_t* s, bool varlen, Plan& p, bool dplr = false,
                                   bool f32_operands = false) {
    kda_status_t st = plan_chunk(s, p);
    if (st != KDA_OK) return st;
    if (dplr && (p.d != 128 || s->gate_per_head != 0)) return KDA_ERR_UNSUPPORTED;
    if (varlen) {
        if (s->batch != 1 || s->num_seqs < 0) return KDA_ERR_INVALID_ARG;
        p.N = s->num_seqs;
        p.tokens = s->seqlen;
        p.max_len = s->max_seqlen > 0 ? s->max_seqlen : s->seqlen;
    } else {
        p.N = s->batch;
        p.tokens = (int64_t)s->batch * s->seqlen;
        p.max_len = s->seqlen;
    }
    if (p.N * (int64_t)s->heads > INT32_MAX / 16) return KDA_ERR_UNSUPPORTED;
    p.max_chunks = (p.max_len + CHUNK - 1) / CHUNK;
    const bool bf16 = enum_code(s->in_dtype) == KDA_DTYPE_BF16;
    p.rec = dplr ? kda::dplr_record_bytes(bf16) : kda::chunk_record_bytes(p.d, bf16 && !f32_operands);
    p.state_bytes = align256((size_t)p.N * s->heads * p.d * p.d * sizeof(float));
    return KDA_OK;
}

// Record bytes of the windowed schedule: every chunk if that fits the record
// budget, else windows of chunks.
static size_t window_record_bytes(const Plan& p, size_t per_chunk) {
    const int64_t all = p.max_chunks > 0 ? p.max_chunks : 1;
    if ((size_t)all * per_chunk <= RECORD_BUDGET) return (size_t)all * per_chunk;
    // two windows of half the record budget, or one of twice the size
    int64_t wc = 2 * (int64_t)(RECORD_BUDGET / 2 / per_chunk);
    // Many (sequence, head) pairs leave few chunks per window inside the budget,
    // and then the per-window launch costs outweigh keeping the records in the
    // last-level cache: windows of at least MIN_WINDOW chunks (records of at most
    // WINDOW_CAP bytes; 512 pairs of the 1M-token batch: 5 -> 32 chunks, 1.3x).
    const int64_t wide = std::min<int64_t>(MIN_WINDOW, (int64_t)(WINDOW_CAP / per_chunk));
    wc = std::min<int64_t>(all, std::max<int64_t>(std::max<int64_t>(wc, wide), 1));
    return (size_t)wc * per_chunk;
}

size_t kda_chunk_fwd_workspace_size(const kda_shape_t* s) {
    Plan p;
    if (!s || chunk_plan_full(s, s->num_seqs > 0, p) != KDA_OK) return 0;
    const size_t per_chunk = (size_t)p.N * s->heads * p.rec;
    if (per_chunk == 0) return p.state_bytes + 256;
    const int64_t all = p.max_chunks > 0 ? p.max_chunks : 1;
    const int64_t units = p.N * s->heads;
    int sc = 0;
    const int G = kda::chunk_segments(p.d, kda::chunk_value_slice(p.d, units), units, p.max_chunks, sc);
    size_t need = G > 0  // sequence-parallel state pass: every record plus three per-segment state blocks
                      ? p.state_bytes + (size_t)all * per_chunk + 3 * segment_bytes(p, s->heads, G)
                      : p.state_bytes + window_record_bytes(p, per_chunk);
    // bf16 inputs: room for one chunk of the fp32-operand records KDA_CHECK=1 may select
    Plan p32;
    if (enum_code(s->in_dtype) == KDA_DTYPE_BF16 && chunk_plan_full(s, s->num_seqs > 0, p32, false, true) == KDA_OK)
        need = std::max(need, p32.state_bytes + (size_t)p32.N * s->heads * p32.rec);
    return need;
}


// The prefill behind kda_chunk_fwd (gate: fp32 log_alpha, layer null) and
// kda_layer_fwd (gate: the layer's bf16 pre-activation).
static kda_status_t chunk_fwd_impl(const kda_shape_t* s, const kda_layer_t* layer, const void* q, const void* k,
                                   const void* v, const float* log_alpha, const float* beta,
                                   const float* init_state, const int32_t* cu_seqlens, void* out,
                                   float* final_state, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                   bool static_scratch = false) {
    Plan p;
    kda_status_t st = chunk_plan_full(s, cu_seqlens != nullptr, p);
    if (st != KDA_OK) return st;
    const int H = s->heads, d = p.d;
    const size_t in_b = dsize(enum_code(s->in_dtype)), out_b = dsize(enum_code(s->out_dtype));
    const size_t tok_bytes = (size_t)p.tokens * H * d;
    const void* gate = layer ? layer->gate : static_cast<const void*>(log_alpha);
    const size_t la_bytes = (s->gate_per_head ? (size_t)p.tokens * H : tok_bytes) * (layer ? 2 : 4);
    const size_t og_bytes = layer && layer->out_gate ? tok_bytes * 2 : 0;
    if (layer) {
        if ((layer->qk_l2norm != 0 && layer->qk_l2norm != 1) || !(layer->l2_eps >= 0.f) ||
            !(layer->rms_eps >= 0.f) || !(layer->l2_eps < 3.0e38f) || !(layer->rms_eps < 3.0e38f))
            return KDA_ERR_INVALID_ARG;
        if ((layer->out_gate && !aligned16(layer->out_gate)) ||
            (layer->norm_weight && !aligned16(layer->norm_weight)))
            return KDA_ERR_INVALID_ARG;
    }
    const size_t state_bytes = (size_t)p.N * H * d * d * 4;
    if (p.tokens > 0) {
        if (!q || !k || !v || !gate || !beta || !out) return KDA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(out))
            return KDA_ERR_INVALID_ARG;
    }
    if (cu_seqlens && !aligned16(cu_seqlens)) return KDA_ERR_INVALID_ARG;
    if ((init_state && !aligned16(init_state)) || (final_state && !aligned16(final_state)))
        return KDA_ERR_INVALID_ARG;
    if (init_state && final_state && init_state != final_state &&
        overlaps(init_state, state_bytes, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    // every input (init_state is compared with final_state above)
    const Range inputs[] = {{q, tok_bytes * in_b},
                            {k, tok_bytes * in_b},
                            {v, tok_bytes * in_b},
                            {gate, la_bytes},
                            {beta, (size_t)p.tokens * H * 4},
                            {cu_seqlens, cu_seqlens ? (size_t)(p.N + 1) * 4 : 0},
                            {layer ? layer->out_gate : nullptr, og_bytes},
                            {layer ? layer->norm_weight : nullptr, (size_t)d * 4}};
    const size_t out_bytes = tok_bytes * out_b;
    if (overlaps_any(out, out_bytes, inputs) || overlaps(out, out_bytes, init_state, state_bytes) ||
        overlaps(out, out_bytes, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if (final_state && overlaps_any(final_state, state_bytes, inputs)) return KDA_ERR_INVALID_ARG;

    size_t per_chunk = (size_t)p.N * H * p.rec;
    if (p.N == 0) return KDA_OK;  // nothing to compute
    if (static_scratch) {  // kda_chunk_fwd_noalloc: the device's static array, once arguments are valid
        if (workspace_bytes < p.state_bytes + per_chunk) return KDA_ERR_WORKSPACE;
        hipError_t e;
        workspace = device_scratch(e);
        if (!workspace) return KDA_ERR_HIP;
    }
    if (!workspace || !aligned16(workspace) || workspace_bytes < p.state_bytes + per_chunk)
        return KDA_ERR_WORKSPACE;
    // the workspace is written by the kernels: it must not overlap any argument
    if (overlaps_any(workspace, workspace_bytes, inputs) || overlaps(workspace, workspace_bytes, out, out_bytes) ||
        overlaps(workspace, workspace_bytes, init_state, state_bytes) ||
        overlaps(workspace, workspace_bytes, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if (cu_seqlens && check_enabled()) {
        kda_status_t cs = check_cu_seqlens(cu_seqlens, p, stream);
        if (cs != KDA_OK) return cs;
    }
    bool f32 = false;
    if (check_enabled() && enum_code(s->in_dtype) == KDA_DTYPE_BF16) {
        float* scratch = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + p.state_bytes);
        kda_status_t rs = needs_f32_operands(v, tok_bytes, init_state, init_state ? state_bytes / 4 : 0, scratch,
                                             stream, f32);
        if (rs != KDA_OK) return rs;
        // the layer's epilogue keeps o in the bf16 output buffer as fp16 until it normalises it
        if (f32 && layer && layer->out_gate && enum_code(s->out_dtype) == KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
        if (f32) {  // the larger fp32 records
            p.rec = kda::chunk_record_bytes(d, false);
            per_chunk = (size_t)p.N * H * p.rec;
            if (workspace_bytes < p.state_bytes + per_chunk) return KDA_ERR_WORKSPACE;
        }
    }
    // Few (sequence, head) pairs and a workspace for every record: the
    // sequence-parallel state pass.  Otherwise one buffer for every chunk if it
    // fits, else windows of chunks.
    const size_t avail = workspace_bytes - p.state_bytes;
    const int64_t all = p.max_chunks > 0 ? p.max_chunks : 1;
    const int bv = kda::chunk_value_slice(d, p.N * H);
    int sc = 0;
    int G = kda::chunk_segments(d, bv, p.N * H, p.max_chunks, sc);
    const size_t segb = G > 0 ? segment_bytes(p, H, G) : 0;
    if (G > 0 && avail < (size_t)all * per_chunk + 3 * segb) G = 0;  // workspace too small: windows
    // grid rows of the chunk-local pass: sequences x chunks of a window <= 65535
    const int64_t wc_max = 65535 / p.N;
    if (wc_max < 1) return KDA_ERR_UNSUPPORTED;
    if (G > 0 && all > wc_max) G = 0;  // the sequence-parallel pass launches every chunk at once
    int64_t wc = ((size_t)all * per_chunk <= avail || G > 0) ? all : (int64_t)(avail / per_chunk);
    if (wc > wc_max) wc = wc_max;
    const int64_t nwin64 = p.max_chunks > 0 ? (p.max_chunks + wc - 1) / wc : 1;
    if (nwin64 > INT32_MAX) return KDA_ERR_UNSUPPORTED;

    kda::ChunkArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.la = log_alpha;
    a.gate_per_head = s->gate_per_head;
    if (layer) {
        a.gate = static_cast<const uint16_t*>(layer->gate);
        a.l2_eps = layer->l2_eps;
        a.out_gate = static_cast<const uint16_t*>(layer->out_gate);
        a.norm_weight = layer->norm_weight;
        a.rms_eps = layer->rms_eps;
    }
    a.beta = beta;
    a.cu = cu_seqlens;
    a.T = s->seqlen;
    a.H = H;
    a.N = (int)p.N;
    a.Wc = (int)wc;
    a.win = 0;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    a.state_buf = final_state ? final_state : reinterpret_cast<float*>(ws);
    a.rec = ws + p.state_bytes;
    a.rec_bytes = p.rec;
    a.init = init_state;
    a.out = out;
    if (G > 0) {
        a.G = G;
        a.Sc = sc;
        unsigned char* sb = a.rec + (size_t)all * per_chunk;
        a.seg_B = reinterpret_cast<float*>(sb);
        a.seg_M = reinterpret_cast<float*>(sb + segb);
        a.seg_init = reinterpret_cast<float*>(sb + 2 * segb);
    }
    hipError_t e = kda::chunk_dispatch(d, enum_code(s->in_dtype) == KDA_DTYPE_BF16, enum_code(s->out_dtype) == KDA_DTYPE_BF16,
                                       layer && layer->qk_l2norm, bv, a, (int)nwin64, stream, f32);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_chunk_fwd(const kda_shape_t* s, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    return chunk_fwd_impl(s, nullptr, q, k, v, log_alpha, beta, init_state, cu_seqlens, out, final_state,
                          workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_fwd_noalloc(const kda_shape_t* s, const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta, const float* init_state,
                                   const int32_t* cu_seqlens, void* out, float* final_state, hipStream_t stream) {
    return chunk_fwd_impl(s, nullptr, q, k, v, log_alpha, beta, init_state, cu_seqlens, out, final_state, nullptr,
                          NOALLOC_SCRATCH_BYTES, stream, /*static_scratch=*/true);
}

size_t kda_dplr_chunk_fwd_workspace_size(const kda_shape_t* s) {
    Plan p;
    if (!s || chunk_plan_full(s, s->num_seqs > 0, p, /*dplr=*/true) != KDA_OK) return 0;
    const size_t per_chunk = (size_t)p.N * s->heads * p.rec;
    if (per_chunk == 0) return p.state_bytes + 256;
    return p.state_bytes + window_record_bytes(p, per_chunk);
}

kda_status_t kda_dplr_chunk_fwd(const kda_shape_t* s, const void* q, const void* k, const void* v, const void* a,
                                const void* b, const float* log_alpha, const float* init_state,
                                const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    Plan p;
    kda_status_t st = chunk_plan_full(s, cu_seqlens != nullptr, p, /*dplr=*/true);
    if (st != KDA_OK) return st;
    const int H = s->heads, d = p.d;
    const size_t in_b = dsize(enum_code(s->in_dtype)), out_b = dsize(enum_code(s->out_dtype));
    const size_t tok_bytes = (size_t)p.tokens * H * d;
    const size_t state_bytes = (size_t)p.N * H * d * d * 4;
    if (p.tokens > 0) {
        if (!q || !k || !v || !a || !b || !log_alpha || !out) return KDA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(a) || !aligned16(b) ||
            !aligned16(log_alpha) || !aligned16(out))
            return KDA_ERR_INVALID_ARG;
    }
    if (cu_seqlens && !aligned16(cu_seqlens)) return KDA_ERR_INVALID_ARG;
    if ((init_state && !aligned16(init_state)) || (final_state && !aligned16(final_state)))
        return KDA_ERR_INVALID_ARG;
    if (init_state && final_state && init_state != final_state &&
        overlaps(init_state, state_bytes, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    const Range inputs[] = {{q, tok_bytes * in_b},
                            {k, tok_bytes * in_b},
                            {v, tok_bytes * in_b},
                            {a, tok_bytes * in_b},
                            {b, tok_bytes * in_b},
                            {log_alpha, tok_bytes * 4},
                            {cu_seqlens, cu_seqlens ? (size_t)(p.N + 1) * 4 : 0}};
    const size_t out_bytes = tok_bytes * out_b;
    if (overlaps_any(out, out_bytes, inputs) || overlaps(out, out_bytes, init_state, state_bytes) ||
        overlaps(out, out_bytes, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if (final_state && overlaps_any(final_state, state_bytes, inputs)) return KDA_ERR_INVALID_ARG;
    const size_t per_chunk = (size_t)p.N * H * p.rec;
    if (p.N == 0) return KDA_OK;  // nothing to compute
    if (!workspace || !aligned16(workspace) || workspace_bytes < p.state_bytes + per_chunk)
        return KDA_ERR_WORKSPACE;
    if (overlaps_any(workspace, workspace_bytes, inputs) || overlaps(workspace, workspace_bytes, out, out_bytes) ||
        overlaps(workspace, workspace_bytes, init_state, state_bytes) ||
        overlaps(workspace, workspace_bytes, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if (cu_seqlens && check_enabled()) {
        kda_status_t cs = check_cu_seqlens(cu_seqlens, p, stream);
        if (cs != KDA_OK) return cs;
    }
    // one record buffer for every chunk if it fits, else windows of chunks
    const size_t avail = workspace_bytes - p.state_bytes;
    const int64_t all = p.max_chunks > 0 ? p.max_chunks : 1;
    const int64_t wc_max = 65535 / p.N;  // grid rows of the chunk-local pass
    if (wc_max < 1) return KDA_ERR_UNSUPPORTED;
    int64_t wc = (size_t)all * per_chunk <= avail ? all : (int64_t)(avail / per_chunk);
    if (wc > wc_max) wc = wc_max;
    const int64_t nwin64 = p.max_chunks > 0 ? (p.max_chunks + wc - 1) / wc : 1;
    if (nwin64 > INT32_MAX) return KDA_ERR_UNSUPPORTED;

    kda::ChunkArgs ca;
    ca.q = q;
    ca.k = k;
    ca.v = v;
    ca.dplr_a = a;
    ca.dplr_b = b;
    ca.la = log_alpha;
    ca.beta = nullptr;
    ca.gate_per_head = 0;
    ca.cu = cu_seqlens;
    ca.T = s->seqlen;
    ca.H = H;
    ca.N = (int)p.N;
    ca.Wc = (int)wc;
    ca.win = 0;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    ca.state_buf = final_state ? final_state : reinterpret_cast<float*>(ws);
    ca.rec = ws + p.state_bytes;
    ca.rec_bytes = p.rec;
    ca.init = init_state;
    ca.out = out;
    const bool in_bf16 = enum_code(s->in_dtype) == KDA_DTYPE_BF16;
    hipError_t e = kda::dplr_dispatch(in_bf16, enum_code(s->out_dtype) == KDA_DTYPE_BF16,
                                      kda::dplr_value_slice(in_bf16, p.N * H), ca, (int)nwin64, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_layer_fwd(const kda_shape_t* s, const kda_layer_t* layer, const void* q, const void* k,
                           const void* v, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    if (!layer) return KDA_ERR_INVALID_ARG;
    return chunk_fwd_impl(s, layer, q, k, v, nullptr, beta, init_state, cu_seqlens, out, final_state, workspace,
                          workspace_bytes, stream);
}

static kda_status_t decode_impl(int32_t batch, int32_t heads, int32_t dk, int32_t dv, int in_dtype,
                                int out_dtype, int32_t gate_per_head, const kda_layer_t* layer,
                                const void* q, const void* k, const void* v, const float* log_alpha,
                                const float* beta, float* state_inout, void* out, hipStream_t stream) {
    if (batch < 0 || heads <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (gate_per_head != 0 && gate_per_head != 1) return KDA_ERR_INVALID_ARG;
    if ((in_dtype != KDA_DTYPE_F32 && in_dtype != KDA_DTYPE_BF16) ||
        (out_dtype != KDA_DTYPE_F32 && out_dtype != KDA_DTYPE_BF16))
        return KDA_ERR_UNSUPPORTED;
    if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (batch == 0) return KDA_OK;
    const int64_t units = (int64_t)batch * heads;
    if (units > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    const void* gate = layer ? layer->gate : static_cast<const void*>(log_alpha);
    if (!q || !k || !v || !gate || !beta || !state_inout || !out) return KDA_ERR_INVALID_ARG;
    if (layer && ((layer->qk_l2norm != 0 && layer->qk_l2norm != 1) || !(layer->l2_eps >= 0.f) ||
                  !(layer->rms_eps >= 0.f) || !(layer->l2_eps < 3.0e38f) || !(layer->rms_eps < 3.0e38f)))
        return KDA_ERR_INVALID_ARG;
    if (!aligned16(state_inout) || !aligned16(out)) return KDA_ERR_INVALID_ARG;
    const size_t vec = (size_t)units * dk;
    const size_t in_b = dsize(in_dtype), out_b = dsize(out_dtype);
    const size_t st_bytes = (size_t)units * dk * dv * 4, out_bytes = vec * out_b;
    const size_t la_bytes = (gate_per_head ? (size_t)units : vec) * (layer ? 2 : 4);
    const size_t og_bytes = layer && layer->out_gate ? vec * 2 : 0;
    const Range inputs[] = {{q, vec * in_b},
                            {k, vec * in_b},
                            {v, vec * in_b},
                            {gate, la_bytes},
                            {beta, (size_t)units * 4},
                            {layer ? layer->out_gate : nullptr, og_bytes},
                            {layer ? layer->norm_weight : nullptr, (size_t)dv * 4}};
    if (overlaps(out, out_bytes, state_inout, st_bytes) || overlaps_any(out, out_bytes, inputs) ||
        overlaps_any(state_inout, st_bytes, inputs))
        return KDA_ERR_INVALID_ARG;
    kda::DecodeLayer L;
    if (layer) {
        L.gate = static_cast<const uint16_t*>(layer->gate);
        L.qk_norm = layer->qk_l2norm;
        L.l2_eps = layer->l2_eps;
        L.out_gate = static_cast<const uint16_t*>(layer->out_gate);
        L.norm_weight = layer->norm_weight;
        L.rms_eps = layer->rms_eps;
    }
    hipError_t e = kda::decode_dispatch((int)units, dk, in_dtype == KDA_DTYPE_BF16, out_dtype == KDA_DTYPE_BF16,
                                        gate_per_head != 0, q, k, v, log_alpha, beta, state_inout, out, L,
                                        stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_decode_step(int32_t batch, int32_t heads, int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                             kda_dtype_t out_dtype, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, float* state_inout, void* out,
                             hipStream_t stream) {
    return decode_impl(batch, heads, dk, dv, enum_code(in_dtype), enum_code(out_dtype), 0, nullptr, q, k, v, log_alpha, beta, state_inout,
                       out, stream);
}

kda_status_t kda_decode_step_head_gate(int32_t batch, int32_t heads, int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                                       kda_dtype_t out_dtype, const void* q, const void* k, const void* v,
                                       const float* log_alpha, const float* beta, float* state_inout, void* out,
                                       hipStream_t stream) {
    return decode_impl(batch, heads, dk, dv, enum_code(in_dtype), enum_code(out_dtype), 1, nullptr, q, k, v, log_alpha, beta, state_inout,
                       out, stream);
}

kda_status_t kda_dplr_decode_step(int32_t batch, int32_t heads, int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                                  kda_dtype_t out_dtype, const void* q, const void* k, const void* v, const void* a,
                                  const void* b, const float* log_alpha, float* state_inout, void* out,
                                  hipStream_t stream) {
    if (batch < 0 || heads <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    const int in_dt = enum_code(in_dtype), out_dt = enum_code(out_dtype);
    if ((in_dt != KDA_DTYPE_F32 && in_dt != KDA_DTYPE_BF16) || (out_dt != KDA_DTYPE_F32 && out_dt != KDA_DTYPE_BF16))
        return KDA_ERR_UNSUPPORTED;
    if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (batch == 0) return KDA_OK;
    const int64_t units = (int64_t)batch * heads;
    if (units > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !a || !b || !log_alpha || !state_inout || !out) return KDA_ERR_INVALID_ARG;
    if (!aligned16(state_inout) || !aligned16(out)) return KDA_ERR_INVALID_ARG;
    const size_t vec = (size_t)units * dk;
    const size_t in_b = dsize(in_dt), out_b = dsize(out_dt);
    const size_t st_bytes = (size_t)units * dk * dv * 4, out_bytes = vec * out_b;
    const Range inputs[] = {{q, vec * in_b}, {k, vec * in_b}, {v, vec * in_b},
                            {a, vec * in_b}, {b, vec * in_b}, {log_alpha, vec * 4}};
    if (overlaps(out, out_bytes, state_inout, st_bytes) || overlaps_any(out, out_bytes, inputs) ||
        overlaps_any(state_inout, st_bytes, inputs))
        return KDA_ERR_INVALID_ARG;
    hipError_t e = kda::dplr_decode_dispatch((int)units, dk, in_dt == KDA_DTYPE_BF16, out_dt == KDA_DTYPE_BF16, q, k,
                                             v, a, b, log_alpha, state_inout, out, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_layer_decode_step(int32_t batch, int32_t heads, int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                                   kda_dtype_t out_dtype, int32_t gate_per_head, const kda_layer_t* layer,
                                   const void* q, const void* k, const void* v, const float* beta,
                                   float* state_inout, void* out, hipStream_t stream) {
    if (!layer) return KDA_ERR_INVALID_ARG;
    return decode_impl(batch, heads, dk, dv, enum_code(in_dtype), enum_code(out_dtype), gate_per_head, layer, q, k, v, nullptr, beta,
                       state_inout, out, stream);
}

// Workspace of the backward: state buffer, the forward records of one record
// window of the recompute (at most the record budget), then per (chunk, head)
// of one backward window the state snapshot, the fp32 backward record, the
// gradient snapshot and dU; with more than one backward window, the states
// entering windows 1, 2, ... and the carried dL/dS.
struct BwdLayout {
    size_t state, rec, snap, brec, dsnap, du, ckpt, dcarry, total;
    int window;      // chunks per record window of the forward recompute
    int bwd_window;  // chunks per sequence held by the per-chunk arrays
    int nbw;         // backward windows
};

// Bytes of per-chunk backward arrays held at once before the backward walks
// its chunks in windows (KDA_BWD_WINDOW=n forces n chunks per window).
constexpr size_t BWD_BUDGET = size_t(24) << 30;

static kda_status_t bwd_layout(const kda_shape_t* s, bool varlen, Plan& p, BwdLayout& l, bool f32 = false) {
    kda_status_t st = chunk_plan_full(s, varlen, p, false, f32);
    if (st != KDA_OK) return st;
    const int64_t all = p.max_chunks > 0 ? p.max_chunks : 1;
    const size_t d = p.d, H = s->heads;
    const size_t per_chunk = (size_t)p.N * H * p.rec;  // forward records of one chunk index
    const size_t per_bwd = (size_t)p.N * H * (kda::bwd_record_bytes(p.d) + (2 * d * d + CHUNK * d) * sizeof(float));
    int64_t rw = per_chunk == 0 ? 1 : std::min<int64_t>(all, std::max<size_t>(1, RECORD_BUDGET / per_chunk));
    int64_t wb = all;
    const char* e = getenv("KDA_BWD_WINDOW");  // read per call
    if (e && atoi(e) > 0) wb = std::min<int64_t>(all, atoi(e));
    else if (per_bwd * all > BWD_BUDGET) wb = std::max<int64_t>(1, (int64_t)(BWD_BUDGET / per_bwd));
    if (p.N > 0) wb = std::min<int64_t>(wb, 65535 / p.N);  // grid rows: sequences x chunks of a window
    if (wb < 1) return KDA_ERR_UNSUPPORTED;
    if (wb < all) {  // several backward windows: each a whole number of record windows
        if (rw > wb) rw = wb;
        else wb = wb / rw * rw;
    }
    l.window = (int)rw;
    l.bwd_window = (int)wb;
    l.nbw = (int)((all + wb - 1) / wb);
    const size_t units = (size_t)p.N * wb * H;
    l.state = 0;
    l.rec = p.state_bytes;
    l.snap = l.rec + align256(per_chunk * rw);
    l.brec = l.snap + align256(units * d * d * 4);
    l.dsnap = l.brec + align256(units * kda::bwd_record_bytes(p.d));
    l.du = l.dsnap + align256(units * d * d * 4);
    l.ckpt = l.du + align256(units * CHUNK * d * 4);
    l.dcarry = l.ckpt + (l.nbw > 1 ? (size_t)(l.nbw - 1) * p.state_bytes : 0);
    l.total = l.dcarry + (l.nbw > 1 ? p.state_bytes : 0) + 256;
    return KDA_OK;
}

size_t kda_chunk_bwd_workspace_size(const kda_shape_t* s) {
    Plan p;
    BwdLayout l;
    if (!s || bwd_layout(s, s->num_seqs > 0, p, l) != KDA_OK) return 0;
    size_t need = l.total;
    // bf16 inputs: also the layout with the fp32-operand records KDA_CHECK=1 may select
    if (enum_code(s->in_dtype) == KDA_DTYPE_BF16 && bwd_layout(s, s->num_seqs > 0, p, l, true) == KDA_OK)
        need = std::max(need, l.total);
    return need;
}

kda_status_t kda_chunk_bwd(const kda_shape_t* s, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, const void* d_out, const float* d_final_state, float* dq,
                           float* dk, float* dv, float* dlog_alpha, float* dbeta, float* d_init_state,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Plan p;
    BwdLayout l;
    kda_status_t st = bwd_layout(s, cu_seqlens != nullptr, p, l);
    if (st != KDA_OK) return st;
    const int H = s->heads, d = p.d;
    const size_t tok = (size_t)p.tokens * H * d;
    const size_t in_b = dsize(enum_code(s->in_dtype)), out_b = dsize(enum_code(s->out_dtype));
    const size_t la_bytes = (s->gate_per_head ? (size_t)p.tokens * H : tok) * 4;
    const size_t st_bytes = (size_t)p.N * H * d * d * 4, tb4 = (size_t)p.tokens * H * 4;
    if (p.tokens > 0) {
        if (!q || !k || !v || !log_alpha || !beta || !d_out || !dq || !dk || !dv || !dlog_alpha || !dbeta)
            return KDA_ERR_INVALID_ARG;
        const void* ptrs[] = {q, k, v, log_alpha, beta, d_out, dq, dk, dv, dlog_alpha, dbeta};
        for (const void* x : ptrs)
            if (!aligned16(x)) return KDA_ERR_INVALID_ARG;
    }
    if ((cu_seqlens && !aligned16(cu_seqlens)) || (init_state && !aligned16(init_state)) ||
        (d_final_state && !aligned16(d_final_state)) || (d_init_state && !aligned16(d_init_state)))
        return KDA_ERR_INVALID_ARG;
    {  // outputs against inputs and one another
        const void* outs[] = {dq, dk, dv, dlog_alpha, dbeta, d_init_state};
        const size_t osz[] = {tok * 4, tok * 4, tok * 4, la_bytes, tb4, st_bytes};
        const void* ins[] = {q, k, v, log_alpha, beta, init_state, cu_seqlens, d_out, d_final_state};
        const size_t isz[] = {tok * in_b, tok * in_b, tok * in_b, la_bytes, tb4, st_bytes,
                              (size_t)(p.N + 1) * 4, tok * out_b, st_bytes};
        for (int i = 0; i < 6; ++i) {
            for (int j = 0; j < 9; ++j)
                if (overlaps(outs[i], osz[i], ins[j], isz[j])) return KDA_ERR_INVALID_ARG;
            for (int j = i + 1; j < 6; ++j)
                if (overlaps(outs[i], osz[i], outs[j], osz[j])) return KDA_ERR_INVALID_ARG;
        }
    }
    if (p.N == 0) return KDA_OK;
    if (cu_seqlens && check_enabled()) {
        kda_status_t cs = check_cu_seqlens(cu_seqlens, p, stream);
        if (cs != KDA_OK) return cs;
    }
    if (!workspace || !aligned16(workspace) || workspace_bytes < l.total) return KDA_ERR_WORKSPACE;
    {  // the workspace is written by the kernels: it must not overlap any argument
        const Range all[] = {{q, tok * in_b},       {k, tok * in_b},         {v, tok * in_b},
                             {log_alpha, la_bytes}, {beta, tb4},             {init_state, st_bytes},
                             {cu_seqlens, cu_seqlens ? (size_t)(p.N + 1) * 4 : 0},
                             {d_out, tok * out_b},  {d_final_state, st_bytes}, {dq, tok * 4},
                             {dk, tok * 4},         {dv, tok * 4},           {dlog_alpha, la_bytes},
                             {dbeta, tb4},          {d_init_state, st_bytes}};
        if (overlaps_any(workspace, workspace_bytes, all)) return KDA_ERR_INVALID_ARG;
    }
    bool f32 = false;
    if (check_enabled() && enum_code(s->in_dtype) == KDA_DTYPE_BF16) {
        float* scratch = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + l.rec);
        kda_status_t rs = needs_f32_operands(v, tok, init_state, init_state ? st_bytes / 4 : 0, scratch, stream, f32);
        if (rs != KDA_OK) return rs;
        if (f32) {  // the recompute with fp32 records: their layout
            if ((st = bwd_layout(s, cu_seqlens != nullptr, p, l, true)) != KDA_OK) return st;
            if (workspace_bytes < l.total) return KDA_ERR_WORKSPACE;
        }
    }
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    kda::BwdArgs b;
    b.f32_records = f32;
    kda::ChunkArgs& a = b.fwd;
    a.q = q;
    a.k = k;
    a.v = v;
    a.la = log_alpha;
    a.gate_per_head = s->gate_per_head;
    a.beta = beta;
    a.cu = cu_seqlens;
    a.T = s->seqlen;
    a.H = H;
    a.N = (int)p.N;
    a.Wc = (int)(p.max_chunks > 0 ? p.max_chunks : 1);
    a.win = 0;
    a.state_buf = reinterpret_cast<float*>(ws + l.state);
    a.rec = ws + l.rec;
    a.rec_bytes = p.rec;
    a.init = init_state;
    a.out = nullptr;
    a.snap = reinterpret_cast<float*>(ws + l.snap);
    b.brec = reinterpret_cast<float*>(ws + l.brec);
    b.snap_window = l.window;
    b.bwd_window = l.bwd_window;
    b.ckpt = l.nbw > 1 ? reinterpret_cast<float*>(ws + l.ckpt) : nullptr;
    b.dcarry = l.nbw > 1 ? reinterpret_cast<float*>(ws + l.dcarry) : nullptr;
    b.dO = d_out;
    b.dfinal = d_final_state;
    b.dsnap = reinterpret_cast<float*>(ws + l.dsnap);
    b.dU = reinterpret_cast<float*>(ws + l.du);
    b.dinit = d_init_state;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.dG = s->gate_per_head ? nullptr : dlog_alpha;
    b.dla_head = s->gate_per_head ? dlog_alpha : nullptr;
    b.dbeta = dbeta;
    hipError_t e = kda::bwd_dispatch(d, enum_code(s->in_dtype) == KDA_DTYPE_BF16, enum_code(s->out_dtype) == KDA_DTYPE_BF16, b,
                                     stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
