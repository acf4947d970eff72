// kda_internal.h -- declarations shared by the kernel files and the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Arguments of one window of the chunked prefill (see kda_chunk.hip).
struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dplr_a = nullptr;  // general DPLR variant: the rank-one vectors a and b
    const void* dplr_b = nullptr;
    const float* la;
    const float* beta;
    const int32_t* cu;  // packed sequence offsets, or null for a dense batch
    int64_t T;          // dense: tokens per sequence
    int H;
    int gate_per_head;  // log_alpha is [tokens, H] (one gate per head) instead of [tokens, H, D]
    int N;       // sequences
    int Wc;      // chunks per sequence per window
    int win;     // window index
    unsigned char* rec;
    size_t rec_bytes;
    const float* init;
    float* state_buf;
    void* out;
    // sequence-parallel state pass: G segments of Sc chunks per sequence, all
    // records in one buffer; per (unit, segment) [D, D] fp32 blocks
    int G = 0;
    int Sc = 0;
    float* seg_B = nullptr;           // end state of each segment from a zero state
    float* seg_M = nullptr;           // transition product of each segment
    float* seg_init = nullptr;        // true initial state of each segment
    // layer prologue and epilogue (null pointers: off)
    const uint16_t* gate = nullptr;       // bf16 gate pre-activation g replacing la: alpha = sigmoid(-g)
    float l2_eps = 0.f;                   // q, k / sqrt(sum of squares + l2_eps) when normalised
    const uint16_t* out_gate = nullptr;   // bf16 [tokens, H, D] output-gate pre-activation
    const float* norm_weight = nullptr;   // fp32 [D] RMSNorm weight, or null for ones
    float rms_eps = 0.f;
    // backward recompute: the state entering every chunk, [sequence][chunk][H][D][D]
    // fp32 with snap_wc chunks per sequence (null: not written); a null `out` skips
    // the outputs
    float* snap = nullptr;
    int snap_wc = 0;
    int snap_j0 = 0;  // chunk index of the snapshot array's first chunk
    // with snap: the chunk's U = Ut - W S_j as the state pass forms it, fp32 [64][D]
    // at snapU + (the snapshot's chunk-head index) * snapU_stride (null: not written)
    float* snapU = nullptr;
    size_t snapU_stride = 0;
};

// Layer prologue and epilogue of one decode step (null pointers: off).
struct DecodeLayer {
    const uint16_t* gate = nullptr;       // bf16 [batch, H, D] or [batch, H]: alpha = sigmoid(-g)
    int qk_norm = 0;
    float l2_eps = 0.f;
    const uint16_t* out_gate = nullptr;   // bf16 [batch, H, D]
    const float* norm_weight = nullptr;
    float rms_eps = 0.f;
};

// Reverse mode of the chunked prefill (kda_backward.hip).  fwd: the forward's
// arguments with Wc = the longest sequence's chunks, rec / state_buf in the
// workspace, snap set and out null.  The backward walks windows of bwd_window
// chunks per sequence from the last to the first; its per-chunk arrays (snap,
// brec, dsnap, dU) hold one such window, indexed [sequence][chunk in window]
// [head].  Each window's forward recompute runs in record windows of
// snap_window chunks (bwd_window is a multiple of it) from the state entering
// the window: the initial state, or a checkpoint stored by a first forward
// pass when there is more than one window.
struct BwdArgs {
    ChunkArgs fwd;
    int snap_window;      // chunks per window of the forward recompute
    int bwd_window;       // chunks per sequence held by the backward's arrays
    float* ckpt;          // [windows - 1][N, H, D, D]: state entering windows 1, 2, ...; null with one window
    float* dcarry;        // [N, H, D, D]: dL/dS entering the window just walked; null with one window
    float* brec;          // fp32 per-(chunk, head) records of the backward
    const void* dO;       // dL/dout, [tokens, H, D] (out dtype)
    const float* dfinal;  // dL/dfinal_state [N, H, D, D] or null
    float* dsnap;         // dL/dS_{j+1} per (chunk, head), [D, D]
    float* dU;            // dL/dU per (chunk, head), [64, D]
    float* dinit;         // dL/dinit_state [N, H, D, D] or null
    float *dq, *dk, *dv;  // [tokens, H, D] fp32
    float* dG;            // [tokens, H, D] fp32: dL/dlog_alpha per channel; null when the gate is per head
    float* dla_head;      // [tokens, H] fp32 when the gate is per head, else null
    float* dbeta;         // [tokens, H] fp32
    bool f32_records = false;  // bf16 inputs: recompute the forward with fp32 operands and records
};
size_t bwd_record_bytes(int d);
hipError_t bwd_dispatch(int d, bool in_bf16, bool dout_bf16, const BwdArgs& b, hipStream_t st);
// The forward recompute of the backward: chunk-local records and, with `snap`,
// the state entering each chunk (a.snap, a.snap_wc chunks per sequence from
// chunk a.snap_j0), for record windows w0 .. w0 + nw - 1 of `window` chunks
// through one record buffer, carrying S through a.state_buf; no outputs.
hipError_t chunk_snapshot_dispatch(int d, bool in_bf16, const ChunkArgs& a, int window, int w0, int nw, bool snap,
                                   hipStream_t st, bool f32_operands = false);

size_t chunk_record_bytes(int d, bool in_bf16);
int chunk_value_slice(int d, int64_t units);
// Segments per sequence for the sequence-parallel state pass (0: windows), and
// the chunks per segment.  KDA_SEGMENTS=0 turns it off, KDA_SEGMENTS=n asks for n.
int chunk_segments(int d, int bv, int64_t units, int64_t max_chunks, int& chunks_per_segment);
// qk_norm: q and k L2-normalised per (token, head) in the chunk-local pass.
// With a.out_gate set, the state pass writes o to `out` (fp16 when out_bf16,
// else fp32) and an epilogue pass after the last window replaces it in place
// by RMSNorm(o) * w * sigmoid(out_gate) (bf16 or fp32).
// f32_operands: bf16 inputs with fp32 matrix-core operands and records (the
// fp32 inputs' kernels reading bf16), for values past the fp16 operands' range.
hipError_t chunk_dispatch(int d, bool in_bf16, bool out_bf16, bool qk_norm, int bv, const ChunkArgs& a, int nwin,
                          hipStream_t st, bool f32_operands = false);
// Largest |x| over n elements (bf16 or fp32; NaN counts as +inf), as one partial
// maximum per block in block_max[0 .. nblocks), nblocks <= 1024.
hipError_t max_abs_dispatch(const void* x, size_t n, bool bf16, float* block_max, int nblocks, hipStream_t st);
// General DPLR variant (dplr_chunk.hip): dk = dv = 128, windows of a.Wc chunks,
// value slices of 16 or 32 columns (16 for fp32 inputs).
size_t dplr_record_bytes(bool in_bf16);
int dplr_value_slice(bool in_bf16, int64_t units);
hipError_t dplr_dispatch(bool in_bf16, bool out_bf16, int bv, const ChunkArgs& a, int nwin, hipStream_t st);
hipError_t decode_dispatch(int units, int d, bool in_bf16, bool out_bf16, bool gate_per_head, const void* q,
                           const void* k, const void* v, const float* la, const float* beta, float* state,
                           void* out, const DecodeLayer& layer, hipStream_t st);
// One step of the general DPLR transition (kda_decode.hip), d in {64, 128}.
hipError_t dplr_decode_dispatch(int units, int d, bool in_bf16, bool out_bf16, const void* q, const void* k,
                                const void* v, const void* a, const void* b, const float* la, float* state,
                                void* out, hipStream_t st);

}  // namespace kda
