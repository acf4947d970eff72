// kda_api.hip -- the extern "C" boundary of libkda: argument validation,
// workspace sizing and kernel launches.  See include/kda.h for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stdlib.h>

#include <mutex>
#include <vector>

#include "../../include/kda.h"

#include "kda_internal.h"

namespace {

constexpr int CHUNK = 64;
// Record budget across the two window buffers: records written by the
// chunk-local pass should still sit in the 256 MB last-level (MALL) cache when
// the state pass reads them.  The chunk-local pass streams its inputs and
// outputs with non-temporal accesses, so records of up to about 230 MB stay
// resident; past that the state pass starts missing.
constexpr size_t RECORD_BUDGET = size_t(220) << 20;
constexpr int64_t MIN_WINDOW = 32;
constexpr size_t WINDOW_CAP = size_t(4) << 30;

// Per-device overlap resources, created on first use and kept for the life of
// the process.  The mutex serialises host-side enqueueing of calls on one device.
struct DeviceResources {
    std::mutex mu;
    bool ready = false;
    kda::Overlap ov;
};
constexpr int MAX_DEVICES = 64;
DeviceResources g_dev[MAX_DEVICES];

DeviceResources* device_resources() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    DeviceResources* r = &g_dev[dev];
    return r;
}

void init_overlap(DeviceResources* r) {
    if (r->ready) return;
    r->ready = true;
    kda::Overlap ov;
    if (hipStreamCreateWithFlags(&ov.side, hipStreamNonBlocking) != hipSuccess) return;
    if (hipEventCreateWithFlags(&ov.local_done, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ov.inter_done[0], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ov.inter_done[1], hipEventDisableTiming) != hipSuccess)
        return;  // resources leak on this rare path; the overlap simply stays off
    r->ov = ov;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

size_t dsize(kda_dtype_t t) { return t == KDA_DTYPE_BF16 ? 2 : 4; }

struct Plan {
    int64_t N, tokens, max_len, max_chunks;
    int d;
    size_t rec, state_bytes;
};

kda_status_t plan_chunk(const kda_shape_t* s, Plan& p) {
    if (!s) return KDA_ERR_INVALID_ARG;
    if (s->heads <= 0 || s->batch <= 0 || s->seqlen < 0 || s->dk <= 0 || s->dv <= 0 || s->max_seqlen < 0)
        return KDA_ERR_INVALID_ARG;
    if ((s->in_dtype != KDA_DTYPE_F32 && s->in_dtype != KDA_DTYPE_BF16) ||
        (s->out_dtype != KDA_DTYPE_F32 && s->out_dtype != KDA_DTYPE_BF16))
        return KDA_ERR_UNSUPPORTED;
    if (s->dk != s->dv || (s->dk != 64 && s->dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (s->gate_per_head != 0 && s->gate_per_head != 1) return KDA_ERR_INVALID_ARG;
    p.d = s->dk;
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status_t st) {
    switch (st) {
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

// Bytes of one per-segment state array [units, G, d, d] fp32 (256-aligned).
static size_t segment_bytes(const Plan& p, int heads, int G) {
    return align256((size_t)p.N * heads * G * p.d * p.d * sizeof(float));
}

static kda_status_t chunk_plan_full(const kda_shape_t* s, bool varlen, Plan& p) {
    kda_status_t st = plan_chunk(s, p);
    if (st != KDA_OK) return st;
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
    p.rec = kda::chunk_record_bytes(p.d, s->in_dtype == KDA_DTYPE_BF16);
    p.state_bytes = align256((size_t)p.N * s->heads * p.d * p.d * sizeof(float));
    return KDA_OK;
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
    if (G > 0)  // sequence-parallel state pass: every record plus three per-segment state blocks
        return p.state_bytes + (size_t)all * per_chunk + 3 * segment_bytes(p, s->heads, G);
    if ((size_t)all * per_chunk <= RECORD_BUDGET) return p.state_bytes + (size_t)all * per_chunk;
    // two windows of half the record budget, or one of twice the size
    int64_t wc = 2 * (int64_t)(RECORD_BUDGET / 2 / per_chunk);
    // Many (sequence, head) pairs leave few chunks per window inside the budget,
    // and then the per-window launch costs outweigh keeping the records in the
    // last-level cache: windows of at least MIN_WINDOW chunks (records of at most
    // WINDOW_CAP bytes; 512 pairs of the 1M-token batch: 5 -> 32 chunks, 1.3x).
    const int64_t wide = std::min<int64_t>(MIN_WINDOW, (int64_t)(WINDOW_CAP / per_chunk));
    wc = std::min<int64_t>(all, std::max<int64_t>(std::max<int64_t>(wc, wide), 1));
    return p.state_bytes + (size_t)wc * per_chunk;
}

// The prefill behind kda_chunk_fwd (gate: fp32 log_alpha, layer null) and
// kda_layer_fwd (gate: the layer's bf16 pre-activation).
static kda_status_t chunk_fwd_impl(const kda_shape_t* s, const kda_layer_t* layer, const void* q, const void* k,
                                   const void* v, const float* log_alpha, const float* beta,
                                   const float* init_state, const int32_t* cu_seqlens, void* out,
                                   float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    kda_status_t st = chunk_plan_full(s, cu_seqlens != nullptr, p);
    if (st != KDA_OK) return st;
    const int H = s->heads, d = p.d;
    const size_t in_b = dsize(s->in_dtype), out_b = dsize(s->out_dtype);
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
    const size_t state_elems = (size_t)p.N * H * d * d;
    if (p.tokens > 0) {
        if (!q || !k || !v || !gate || !beta || !out) return KDA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(out))
            return KDA_ERR_INVALID_ARG;
    }
    if (cu_seqlens && !aligned16(cu_seqlens)) return KDA_ERR_INVALID_ARG;
    if ((init_state && !aligned16(init_state)) || (final_state && !aligned16(final_state)))
        return KDA_ERR_INVALID_ARG;
    if (init_state && final_state && init_state != final_state &&
        overlaps(init_state, state_elems * 4, final_state, state_elems * 4))
        return KDA_ERR_INVALID_ARG;
    const size_t out_bytes = tok_bytes * out_b;
    if (overlaps(out, out_bytes, q, tok_bytes * in_b) || overlaps(out, out_bytes, k, tok_bytes * in_b) ||
        overlaps(out, out_bytes, v, tok_bytes * in_b) || overlaps(out, out_bytes, gate, la_bytes) ||
        (layer && overlaps(out, out_bytes, layer->out_gate, og_bytes)) ||
        (layer && overlaps(out, out_bytes, layer->norm_weight, (size_t)d * 4)) ||
        overlaps(out, out_bytes, beta, (size_t)p.tokens * H * 4) ||
        overlaps(out, out_bytes, init_state, state_elems * 4) ||
        overlaps(out, out_bytes, final_state, state_elems * 4))
        return KDA_ERR_INVALID_ARG;
    if (final_state && (overlaps(final_state, state_elems * 4, q, tok_bytes * in_b) ||
                        overlaps(final_state, state_elems * 4, k, tok_bytes * in_b) ||
                        overlaps(final_state, state_elems * 4, v, tok_bytes * in_b)))
        return KDA_ERR_INVALID_ARG;

    const size_t per_chunk = (size_t)p.N * H * p.rec;
    if (p.N == 0) return KDA_OK;  // nothing to compute
    if (cu_seqlens) {
        const char* chk = getenv("KDA_CHECK");
        if (chk && chk[0] == '1') {
            kda_status_t cs = check_cu_seqlens(cu_seqlens, p, static_cast<hipStream_t>(stream));
            if (cs != KDA_OK) return cs;
        }
    }
    if (!workspace || !aligned16(workspace) || workspace_bytes < p.state_bytes + per_chunk)
        return KDA_ERR_WORKSPACE;
    // KDA_OVERLAP=1 runs the chunk-local pass of the next window concurrently with the
    // state pass of the current one (two record buffers, an auxiliary stream).  Off by
    // default: on MI355X the concurrent local pass slows the latency-bound state chain
    // more than it saves.
    const char* ov_env = getenv("KDA_OVERLAP");  // read per call (cheap next to any launch)
    const bool overlap_enabled = ov_env && ov_env[0] == '1';
    // Few (sequence, head) pairs and a workspace for every record: the
    // sequence-parallel state pass.  Otherwise one buffer for every chunk if it
    // fits, else windows of chunks.
    const size_t avail = workspace_bytes - p.state_bytes;
    const int64_t all = p.max_chunks > 0 ? p.max_chunks : 1;
    const int bv = kda::chunk_value_slice(d, p.N * H);
    int sc = 0;
    int G = overlap_enabled ? 0 : kda::chunk_segments(d, bv, p.N * H, p.max_chunks, sc);
    const size_t segb = G > 0 ? segment_bytes(p, H, G) : 0;
    if (G > 0 && avail < (size_t)all * per_chunk + 3 * segb) G = 0;  // workspace too small: windows
    // grid rows of the chunk-local pass: sequences x chunks of a window <= 65535
    const int64_t wc_max = 65535 / p.N;
    if (wc_max < 1) return KDA_ERR_UNSUPPORTED;
    if (G > 0 && all > wc_max) G = 0;  // the sequence-parallel pass launches every chunk at once
    int64_t wc;
    bool two = false;
    if ((size_t)all * per_chunk <= avail || G > 0) {
        wc = all;
    } else if (overlap_enabled && avail >= 2 * per_chunk) {
        wc = (int64_t)(avail / 2 / per_chunk);
        two = true;
    } else {
        wc = (int64_t)(avail / per_chunk);
    }
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
    kda::Overlap ov;  // defaults: everything on the caller's stream
    DeviceResources* res = two && nwin64 > 1 ? device_resources() : nullptr;
    std::unique_lock<std::mutex> lock;
    if (res) {
        lock = std::unique_lock<std::mutex>(res->mu);
        init_overlap(res);
        ov = res->ov;
        ov.buffer_bytes = (size_t)wc * per_chunk;
    }
    hipError_t e = kda::chunk_dispatch(d, s->in_dtype == KDA_DTYPE_BF16, s->out_dtype == KDA_DTYPE_BF16,
                                       layer && layer->qk_l2norm, bv, a, (int)nwin64, ov,
                                       static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_chunk_fwd(const kda_shape_t* s, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(s, nullptr, q, k, v, log_alpha, beta, init_state, cu_seqlens, out, final_state,
                          workspace, workspace_bytes, stream);
}

kda_status_t kda_layer_fwd(const kda_shape_t* s, const kda_layer_t* layer, const void* q, const void* k,
                           const void* v, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!layer) return KDA_ERR_INVALID_ARG;
    return chunk_fwd_impl(s, layer, q, k, v, nullptr, beta, init_state, cu_seqlens, out, final_state, workspace,
                          workspace_bytes, stream);
}

static kda_status_t decode_impl(int32_t batch, int32_t heads, int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                                kda_dtype_t out_dtype, int32_t gate_per_head, const kda_layer_t* layer,
                                const void* q, const void* k, const void* v, const float* log_alpha,
                                const float* beta, float* state_inout, void* out, void* stream) {
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
    if (overlaps(out, out_bytes, state_inout, st_bytes) || overlaps(out, out_bytes, q, vec * in_b) ||
        overlaps(out, out_bytes, k, vec * in_b) || overlaps(out, out_bytes, v, vec * in_b) ||
        overlaps(out, out_bytes, gate, la_bytes) || overlaps(out, out_bytes, beta, (size_t)units * 4) ||
        overlaps(state_inout, st_bytes, q, vec * in_b) || overlaps(state_inout, st_bytes, k, vec * in_b) ||
        overlaps(state_inout, st_bytes, v, vec * in_b) || overlaps(state_inout, st_bytes, gate, la_bytes) ||
        overlaps(state_inout, st_bytes, beta, (size_t)units * 4) ||
        (layer && (overlaps(out, out_bytes, layer->out_gate, og_bytes) ||
                   overlaps(out, out_bytes, layer->norm_weight, (size_t)dv * 4) ||
                   overlaps(state_inout, st_bytes, layer->out_gate, og_bytes) ||
                   overlaps(state_inout, st_bytes, layer->norm_weight, (size_t)dv * 4))))
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
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_decode_step(int32_t batch, int32_t heads, int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                             kda_dtype_t out_dtype, int32_t gate_per_head, const void* q, const void* k,
                             const void* v, const float* log_alpha, const float* beta, float* state_inout,
                             void* out, void* stream) {
    return decode_impl(batch, heads, dk, dv, in_dtype, out_dtype, gate_per_head, nullptr, q, k, v, log_alpha, beta,
                       state_inout, out, stream);
}

kda_status_t kda_layer_decode_step(int32_t batch, int32_t heads, int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                                   kda_dtype_t out_dtype, int32_t gate_per_head, const kda_layer_t* layer,
                                   const void* q, const void* k, const void* v, const float* beta,
                                   float* state_inout, void* out, void* stream) {
    if (!layer) return KDA_ERR_INVALID_ARG;
    return decode_impl(batch, heads, dk, dv, in_dtype, out_dtype, gate_per_head, layer, q, k, v, nullptr, beta,
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

static kda_status_t bwd_layout(const kda_shape_t* s, bool varlen, Plan& p, BwdLayout& l) {
    kda_status_t st = chunk_plan_full(s, varlen, p);
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
    return l.total;
}

kda_status_t kda_chunk_bwd(const kda_shape_t* s, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, const void* d_out, const float* d_final_state, float* dq,
                           float* dk, float* dv, float* dlog_alpha, float* dbeta, float* d_init_state,
                           void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    BwdLayout l;
    kda_status_t st = bwd_layout(s, cu_seqlens != nullptr, p, l);
    if (st != KDA_OK) return st;
    const int H = s->heads, d = p.d;
    const size_t tok = (size_t)p.tokens * H * d;
    const size_t in_b = dsize(s->in_dtype), out_b = dsize(s->out_dtype);
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
    if (cu_seqlens) {
        const char* chk = getenv("KDA_CHECK");
        if (chk && chk[0] == '1') {
            kda_status_t cs = check_cu_seqlens(cu_seqlens, p, static_cast<hipStream_t>(stream));
            if (cs != KDA_OK) return cs;
        }
    }
    if (!workspace || !aligned16(workspace) || workspace_bytes < l.total) return KDA_ERR_WORKSPACE;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    kda::BwdArgs b;
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
    hipError_t e = kda::bwd_dispatch(d, s->in_dtype == KDA_DTYPE_BF16, s->out_dtype == KDA_DTYPE_BF16, b,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
