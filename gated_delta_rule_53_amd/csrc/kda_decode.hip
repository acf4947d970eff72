// kda_decode.hip -- fused one-token KDA update, memory-bound state streaming.
//
// Per (sequence, head) the update ("Kimi Linear" page, "Kimi Delta Attention"
// with the delta-rule read/correct/write of "Background: from the delta rule
// to gated DeltaNet") is evaluated column by column of the dk x dv state:
//     S'_{cj} = alpha_c S_{cj}                       (decay, alpha = exp(log_alpha))
//     p_j     = sum_c k_c S'_{cj}                    (prediction)
//     u_j     = beta (v_j - p_j)                     (correction)
//     S_{cj}  = S'_{cj} + k_c u_j                    (write)
//     o_j     = sum_c q_c S_{cj} = sum_c q_c S'_{cj} + (q . k) u_j
// so the state is read once and written once.  One 256-thread workgroup per
// (sequence, head); thread t owns columns 4*(t % CG) .. +3 and a run of RPT
// rows, loading the state as float4 (a wave covers whole 512-byte rows, fully
// coalesced).  The three dot products over c are reduced with a cross-lane
// shuffle inside the wave and through LDS across the four waves, in a fixed
// order, so results are deterministic.
//
// Layer prologue and epilogue ("Kimi Delta Attention" section: the head
// L2-normalises q and k, takes its per-channel decay from a projection output
// and passes o through a head-wise RMSNorm and a sigmoid output gate), each
// switched on by the DecodeLayer argument: q, k / sqrt(sum of squares + eps);
// alpha = sigmoid(-g) = 1 / (1 + e^g) from the bf16 pre-activation g; and
// y = o / sqrt(mean(o^2) + eps) * w * sigmoid(z) over the dv outputs of the
// (sequence, head), which one wave holds.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Five waves per SIMD (96 registers) rather than four: about 1% faster at 256 x 32 units.
// LAYER = false compiles the layer's prologue and epilogue out of the plain operator's
// kernel (92 registers; 179.3 against 180.9 us per step at 256 x 32 units).
template <int D, typename IT, typename OUT, bool LAYER>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) decode_kernel(const IT* __restrict__ q, const IT* __restrict__ k,
                                                     const IT* __restrict__ v,
                                                     const float* __restrict__ log_alpha,
                                                     const float* __restrict__ beta, float* __restrict__ state,
                                                     OUT* __restrict__ out, int gate_per_head, DecodeLayer L) {
    constexpr int CG = D / 4;       // float4 column groups
    constexpr int RG = 256 / CG;    // row groups
    constexpr int RPT = D / RG;     // rows per thread
    constexpr int GPW = 64 / CG;    // row groups per wave
    static_assert(CG * RG == 256 && RPT * RG == D && GPW >= 1, "decode tiling");

    const int unit = blockIdx.x;  // sequence * heads + head
    const int t = threadIdx.x;
    const int jg = t % CG, rg = t / CG;
    const int lane = t & 63, wave = t >> 6;

    float* S_base = state + (size_t)unit * D * D;
    // the state is streamed once per step: non-temporal accesses keep it from
    // displacing other data in L2 and the last-level cache
    floatx4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        S[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(S_base + (size_t)(rg * RPT + i) * D + 4 * jg));

    __shared__ float s_alpha[D], s_k[D], s_q[D], s_v[D];
    __shared__ float s_red[4][CG][9];
    __shared__ float s_nrm[2][D / 64];
    const size_t vec = (size_t)unit * D;
    float kt = 0.f, qt = 0.f;
    if (t < D) {
        if (LAYER && L.gate) {
            const float g = bf16_bits_to_f32(L.gate[gate_per_head ? (size_t)unit : vec + t]);
            s_alpha[t] = __builtin_amdgcn_rcpf(1.f + fast_exp(g));
        } else {
            s_alpha[t] = fast_exp(gate_per_head ? log_alpha[unit] : log_alpha[vec + t]);
        }
        kt = to_f32(k[vec + t]);
        qt = to_f32(q[vec + t]);
        s_v[t] = to_f32(v[vec + t]);
    }
    if (LAYER && L.qk_norm) {
        // sums of squares over the D channels: inside each wave, then across the D / 64 waves
        float sk = kt * kt, sq = qt * qt;
#pragma unroll
        for (int off = 1; off < 64; off *= 2) {
            sk += __shfl_xor(sk, off);
            sq += __shfl_xor(sq, off);
        }
        if (lane == 0 && wave < D / 64) {
            s_nrm[0][wave] = sk;
            s_nrm[1][wave] = sq;
        }
        __syncthreads();
        sk = 0.f;
        sq = 0.f;
#pragma unroll
        for (int w = 0; w < D / 64; ++w) {
            sk += s_nrm[0][w];
            sq += s_nrm[1][w];
        }
        kt *= __builtin_amdgcn_rsqf(sk + L.l2_eps);
        qt *= __builtin_amdgcn_rsqf(sq + L.l2_eps);
    }
    if (t < D) {
        s_k[t] = kt;
        s_q[t] = qt;
    }
    const float b = beta[unit];
    __syncthreads();

    // decay, then partial dot products over this thread's rows
    float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg * RPT + i;
        const float a = s_alpha[c], kc = s_k[c], qc = s_q[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            S[i][e] *= a;
            p[e] += kc * S[i][e];
            r[e] += qc * S[i][e];
        }
        qk += qc * kc;
    }
    // reduce over the row groups inside the wave (lanes with the same column group)
#pragma unroll
    for (int off = CG; off < 64; off *= 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] += __shfl_xor(p[e], off);
            r[e] += __shfl_xor(r[e], off);
        }
        qk += __shfl_xor(qk, off);
    }
    if (lane < CG) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s_red[wave][jg][e] = p[e];
            s_red[wave][jg][4 + e] = r[e];
        }
        s_red[wave][jg][8] = qk;
    }
    __syncthreads();
    float pp[4], rr[4], qq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pp[e] = 0.f;
        rr[e] = 0.f;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pp[e] += s_red[w][jg][e];
            rr[e] += s_red[w][jg][4 + e];
        }
        qq += s_red[w][jg][8];
    }
    float u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = b * (s_v[4 * jg + e] - pp[e]);

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kc = s_k[rg * RPT + i];
        floatx4 n;
#pragma unroll
        for (int e = 0; e < 4; ++e) n[e] = S[i][e] + kc * u[e];
        __builtin_nontemporal_store(n, reinterpret_cast<floatx4*>(S_base + (size_t)(rg * RPT + i) * D + 4 * jg));
    }
    if (rg == 0) {  // lanes 0 .. CG-1 of wave 0 hold the D outputs, four each
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = rr[e] + qq * u[e];
        if (LAYER && L.out_gate) {
            float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
            for (int off = 1; off < CG; off *= 2) ss += __shfl_xor(ss, off);
            const float rs = __builtin_amdgcn_rsqf(ss * (1.f / D) + L.rms_eps);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * jg + e;
                const float z = bf16_bits_to_f32(L.out_gate[vec + j]);
                const float w = L.norm_weight ? L.norm_weight[j] : 1.f;
                o[e] = o[e] * rs * w * __builtin_amdgcn_rcpf(1.f + fast_exp(-z));
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) out[vec + 4 * jg + e] = from_f32<OUT>(o[e]);
    }
}

// One recurrent step of the general DPLR transition KDA constrains ("Kimi Linear"
// page, "The constrained DPLR form and the chunkwise algorithm"), with the
// rank-one term reading the state before the token's decay:
//     w_j    = sum_c b_c S_{cj}
//     S_{cj} = alpha_c S_{cj} - a_c w_j + k_c v_j
//     o_j    = sum_c q_c S_{cj} = sum_c q_c alpha_c S_{cj}^{old} - (q . a) w_j + (q . k) v_j
// Same tiling as decode_kernel: the state is read once and written once, the two
// column sums and the two dot products reduced in a fixed order (deterministic).
// Four waves per SIMD: at five (96 registers) the two extra vectors spill.
template <int D, typename IT, typename OUT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
dplr_decode_kernel(const IT* __restrict__ q, const IT* __restrict__ k, const IT* __restrict__ v,
                   const IT* __restrict__ a, const IT* __restrict__ b, const float* __restrict__ log_alpha,
                   float* __restrict__ state, OUT* __restrict__ out) {
    constexpr int CG = D / 4;       // float4 column groups
    constexpr int RG = 256 / CG;    // row groups
    constexpr int RPT = D / RG;     // rows per thread
    static_assert(CG * RG == 256 && RPT * RG == D && 64 / CG >= 1, "decode tiling");

    const int unit = blockIdx.x;  // sequence * heads + head
    const int t = threadIdx.x;
    const int jg = t % CG, rg = t / CG;
    const int lane = t & 63, wave = t >> 6;

    float* S_base = state + (size_t)unit * D * D;
    floatx4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        S[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(S_base + (size_t)(rg * RPT + i) * D + 4 * jg));

    __shared__ float s_alpha[D], s_a[D], s_b[D], s_k[D], s_q[D], s_v[D];
    __shared__ float s_red[4][CG][11];
    const size_t vec = (size_t)unit * D;
    if (t < D) {
        s_alpha[t] = fast_exp(log_alpha[vec + t]);
        s_a[t] = to_f32(a[vec + t]);
        s_b[t] = to_f32(b[vec + t]);
        s_k[t] = to_f32(k[vec + t]);
        s_q[t] = to_f32(q[vec + t]);
        s_v[t] = to_f32(v[vec + t]);
    }
    __syncthreads();

    // partial column sums over this thread's rows: b^T S and (q o alpha)^T S, both of the old
    // state, and the thread's share of q . a and q . k
    float w[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f}, qa = 0.f, qk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg * RPT + i;
        const float bc = s_b[c], qac = s_q[c] * s_alpha[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] += bc * S[i][e];
            r[e] += qac * S[i][e];
        }
        qa += s_q[c] * s_a[c];
        qk += s_q[c] * s_k[c];
    }
#pragma unroll
    for (int off = CG; off < 64; off *= 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] += __shfl_xor(w[e], off);
            r[e] += __shfl_xor(r[e], off);
        }
        qa += __shfl_xor(qa, off);
        qk += __shfl_xor(qk, off);
    }
    if (lane < CG) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s_red[wave][jg][e] = w[e];
            s_red[wave][jg][4 + e] = r[e];
        }
        s_red[wave][jg][8] = qa;
        s_red[wave][jg][9] = qk;
    }
    __syncthreads();
    float ww[4], rr[4], sqa = 0.f, sqk = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ww[e] = 0.f;
        rr[e] = 0.f;
    }
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ww[e] += s_red[w2][jg][e];
            rr[e] += s_red[w2][jg][4 + e];
        }
        sqa += s_red[w2][jg][8];
        sqk += s_red[w2][jg][9];
    }
    float vj[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vj[e] = s_v[4 * jg + e];

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg * RPT + i;
        const float al = s_alpha[c], ac = s_a[c], kc = s_k[c];
        floatx4 n;
#pragma unroll
        for (int e = 0; e < 4; ++e) n[e] = al * S[i][e] - ac * ww[e] + kc * vj[e];
        __builtin_nontemporal_store(n, reinterpret_cast<floatx4*>(S_base + (size_t)(rg * RPT + i) * D + 4 * jg));
    }
    if (rg == 0) {  // lanes 0 .. CG-1 of wave 0 hold the D outputs, four each
#pragma unroll
        for (int e = 0; e < 4; ++e) out[vec + 4 * jg + e] = from_f32<OUT>(rr[e] - sqa * ww[e] + sqk * vj[e]);
    }
}

template <int D, typename IT, typename OUT>
hipError_t launch_dplr_decode(int units, const void* q, const void* k, const void* v, const void* a, const void* b,
                              const float* la, float* state, void* out, hipStream_t st) {
    hipLaunchKernelGGL((dplr_decode_kernel<D, IT, OUT>), dim3(units), dim3(256), 0, st,
                       static_cast<const IT*>(q), static_cast<const IT*>(k), static_cast<const IT*>(v),
                       static_cast<const IT*>(a), static_cast<const IT*>(b), la, state, static_cast<OUT*>(out));
    return hipGetLastError();
}

hipError_t dplr_decode_dispatch(int units, int d, bool in_bf16, bool out_bf16, const void* q, const void* k,
                                const void* v, const void* a, const void* b, const float* la, float* state,
                                void* out, hipStream_t st) {
#define KDA_DDEC(DD, IT, OT) return launch_dplr_decode<DD, IT, OT>(units, q, k, v, a, b, la, state, out, st)
    if (d == 128) {
        if (in_bf16) {
            if (out_bf16) KDA_DDEC(128, bf16_t, bf16_t);
            KDA_DDEC(128, bf16_t, float);
        }
        if (out_bf16) KDA_DDEC(128, float, bf16_t);
        KDA_DDEC(128, float, float);
    }
    if (in_bf16) {
        if (out_bf16) KDA_DDEC(64, bf16_t, bf16_t);
        KDA_DDEC(64, bf16_t, float);
    }
    if (out_bf16) KDA_DDEC(64, float, bf16_t);
    KDA_DDEC(64, float, float);
#undef KDA_DDEC
}

template <int D, typename IT, typename OUT>
hipError_t launch_decode(int units, bool gph, const void* q, const void* k, const void* v, const float* la,
                         const float* beta, float* state, void* out, const DecodeLayer& L, hipStream_t st) {
    if (L.gate || L.qk_norm || L.out_gate)
        hipLaunchKernelGGL((decode_kernel<D, IT, OUT, true>), dim3(units), dim3(256), 0, st,
                           static_cast<const IT*>(q), static_cast<const IT*>(k), static_cast<const IT*>(v), la,
                           beta, state, static_cast<OUT*>(out), gph ? 1 : 0, L);
    else
        hipLaunchKernelGGL((decode_kernel<D, IT, OUT, false>), dim3(units), dim3(256), 0, st,
                           static_cast<const IT*>(q), static_cast<const IT*>(k), static_cast<const IT*>(v), la,
                           beta, state, static_cast<OUT*>(out), gph ? 1 : 0, L);
    return hipGetLastError();
}

hipError_t decode_dispatch(int units, int d, bool in_bf16, bool out_bf16, bool gate_per_head, const void* q,
                           const void* k, const void* v, const float* la, const float* beta, float* state,
                           void* out, const DecodeLayer& layer, hipStream_t st) {
#define KDA_DEC(DD, IT, OT) \
    return launch_decode<DD, IT, OT>(units, gate_per_head, q, k, v, la, beta, state, out, layer, st)
    if (d == 128) {
        if (in_bf16) {
            if (out_bf16) KDA_DEC(128, bf16_t, bf16_t);
            KDA_DEC(128, bf16_t, float);
        }
        if (out_bf16) KDA_DEC(128, float, bf16_t);
        KDA_DEC(128, float, float);
    }
    if (in_bf16) {
        if (out_bf16) KDA_DEC(64, bf16_t, bf16_t);
        KDA_DEC(64, bf16_t, float);
    }
    if (out_bf16) KDA_DEC(64, float, bf16_t);
    KDA_DEC(64, float, float);
#undef KDA_DEC
}

}  // namespace kda
