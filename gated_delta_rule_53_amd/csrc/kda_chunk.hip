// kda_chunk.hip -- chunked KDA prefill on gfx950.
//
// The chunked algorithm ("Kimi Linear" page, "The constrained DPLR form and
// the chunkwise algorithm"): split each sequence into 64-token chunks, fold the
// per-token corrections of a chunk into a WY form through the UT transform
// (I + A)^-1, run recurrently between chunks and in parallel inside each.
// Because KDA ties both low-rank vectors of its DPLR transition to the key,
// the per-channel gate factors out of every product as a diagonal scaling of
// keys and queries; that is what lets all products below run on matrix cores.
//
// Notation for one (sequence, head) and one chunk of n <= 64 tokens, rows r
// and columns i indexing tokens, c key channels, j value channels;
// G_r = sum_{t<=r} log_alpha_t (chunk-local, per channel):
//   Atil[r,i] = beta_r sum_c k_rc k_ic e^{G_rc - G_ic}      (i < r)
//   P[r,i]    =        sum_c q_rc k_ic e^{G_rc - G_ic}      (i <= r)
//   T         = (I + Atil)^-1
//   W  = T diag(beta) (K e^G),    Ut = T diag(beta) V
//   Qg = Q e^G,   Kh = K e^{G_last - G},   gamma = e^{G_last}
// and between chunks, with the fp32 state S (dk x dv):
//   U = Ut - W S;   O = Qg S + P U;   S <- Diag(gamma) S + Kh^T U.
//
// Two kernels per window of chunks:
//   chunk_local_kernel  one workgroup per (chunk, head): all of the above that
//                       does not depend on S, written to a per-chunk record;
//   chunk_inter_kernel  one workgroup per (sequence, head, slice of BV value
//                       columns): walks the chunks in order carrying S.
// The value columns of S never interact (each column is its own recurrence),
// which is what makes the slice split exact.
//
// Numerics.  Gate products are formed as products of alpha = e^{log_alpha}
// taken over index ranges, never as differences of cumulative sums, so no
// factor overflows: off-diagonal 16x16 sub-blocks use the first row of the
// row block as anchor (both factors <= 1), diagonal sub-blocks use their
// ninth row (factors bounded by eight tokens of decay).  Matrix-core operands
// are fp16 for bf16 inputs and fp32 for fp32 inputs; accumulation, the UT
// inverse and the state are fp32.
#include "kda_chunk_common.h"

#include <stdlib.h>

#include <algorithm>
#include <type_traits>

namespace kda {
// Per-chunk record layout (bytes); OT is the matrix-core operand type.
template <int D, typename OT>
struct Rec {
    static constexpr size_t W = 0;                                        // OT 64 x D, fragment order
    static constexpr size_t QG = align256(W + CH * D * sizeof(OT));       // OT 64 x D, fragment order
    static constexpr size_t KHT = align256(QG + CH * D * sizeof(OT));     // OT D x 64, fragment order
    static constexpr size_t P = align256(KHT + CH * D * sizeof(OT));      // OT 64 x 64, fragment order
    static constexpr size_t UT = align256(P + CH * CH * sizeof(OT));      // OT [4 row tiles][D][16 rows]
    static constexpr size_t GAM = align256(UT + CH * D * sizeof(OT));     // f32 [D]
    static constexpr size_t BYTES = align256(GAM + D * sizeof(float));
};

// ---------------------------------------------------------------------------
// chunk-local kernel
// ---------------------------------------------------------------------------
// One workgroup of 4*D threads per (head, chunk); thread t owns the two
// adjacent key channels 2*(t % (D/2)) and +1 over the eight rows of half-block
// t / (D/2) (rows 8*(t/(D/2)) .. +7).  Every global load is issued first and
// the barriers that precede the first use of k, q and v order LDS only, so
// those loads stay in flight while the gate products are formed.  LDS regions:
//   R0  half-block gate products (exchanged once), then the operand rows of
//       the Atil / P sub-block products, later T (fp32) and the channel-major
//       right-hand sides of W and Ut;
//   R1  Atil (fp32), later T as a matrix-core operand;
//   R2  P staged as the record stores it;
//   R3  beta.
template <int D, typename OT>
struct LocalCfg {
    static constexpr int NT = 4 * D;
    static constexpr int NW = NT / 64;
    static constexpr int PD = Pad<OT>::v;
    static constexpr int DP = D + PD;   // pitch of [row][channel] operand rows (OT)
    static constexpr int DP32 = D + 4;  // pitch of fp32 diagonal-block operand rows
    static constexpr int KP = CH + PD;  // pitch of [channel][token] rows (OT)
    static constexpr int AP = CH + 1;   // pitch of fp32 [64][64] matrices
    static constexpr bool F16 = sizeof(OT) == 2;
    static constexpr size_t SZ_OP = 192 * DP * sizeof(OT);
    static constexpr size_t SZ_KT = (size_t)D * KP * sizeof(OT);
    static constexpr size_t SZ_F = (size_t)CH * AP * sizeof(float);
    static constexpr size_t OFF_KG = F16 ? 0 : SZ_F;          // in R0, after the T phase
    static constexpr size_t R1 = align256(SZ_OP);
    static constexpr size_t R2 = R1 + SZ_F;
    static constexpr size_t R3 = R2 + (size_t)CH * CH * sizeof(OT);
    static constexpr size_t SMEM = R3 + CH * sizeof(float);
    static_assert(24 * D * sizeof(float) <= SZ_OP, "half-block products must fit R0");
    static_assert(OFF_KG + 2 * SZ_KT <= SZ_OP, "W/Ut right-hand sides must fit R0");
    static_assert(!F16 || 96 * DP32 * sizeof(float) <= SZ_OP, "fp32 diagonal operands must fit R0");
    static_assert(!F16 || (size_t)CH * KP * sizeof(OT) <= SZ_F, "T operand must fit R1");
};


// The diagonal sub-blocks split e^{G_r - G_i} into a row factor and a column
// factor about an anchor row; they switch to fp32 operands when an fp16 operand
// could overflow, or when a factor exceeds F16_FACTOR_LIMIT: its partner factor is
// then below 1/256, the partner operand may be an fp16 subnormal, and that
// operand's absolute rounding error times the large factor would no longer be
// negligible next to the entry being formed (it stays below 2^-17 of |k_r k_i|).
// With fp32 operands (fp32 inputs) only the range matters: a factor up to 2^64
// keeps its partner's absolute error below 2^64 times the smallest subnormal.
// Past either limit the sub-blocks are formed in the multi-level form below,
// whose factors never exceed 1, so no gate value is out of range.
constexpr float F16_OPERAND_LIMIT = 6.0e4f;
constexpr float F16_FACTOR_LIMIT = 256.f;
constexpr float F32_FACTOR_LIMIT = 1.8446744e19f;  // 2^64

// The chunk-local work of one workgroup.  WIDE = false: the diagonal sub-blocks in
// the single-anchor form; it returns false, before storing anything, when their
// factors leave that form's range (uniformly over the workgroup).  WIDE = true:
// the multi-level form, valid for every gate.  The kernel runs the second only
// after the first declined, so the rarely taken form adds nothing to the
// registers of the common one.
template <int D, typename IT, typename OT, bool QKN, bool GPRE, bool WIDE>
__device__ __forceinline__ bool chunk_local_body(const ChunkArgs& a, unsigned char* smem, int bx, int by, int tid) {
    using C = LocalCfg<D, OT>;
    using R = Rec<D, OT>;
    using FO = FragOrder<OT>;
    OT* sOp = reinterpret_cast<OT*>(smem);
    float* sOp32 = reinterpret_cast<float*>(smem);
    float* sT = reinterpret_cast<float*>(smem);
    float* sX = reinterpret_cast<float*>(smem);  // half-block gate products (aliases R0 before phase A)
    OT* sKgT = reinterpret_cast<OT*>(smem + C::OFF_KG);
    OT* sVbT = reinterpret_cast<OT*>(smem + C::OFF_KG + C::SZ_KT);
    float* sAt = reinterpret_cast<float*>(smem + C::R1);
    OT* sTh = C::F16 ? reinterpret_cast<OT*>(smem + C::R1) : reinterpret_cast<OT*>(smem);
    constexpr int THP = C::F16 ? C::KP : C::AP;  // pitch of the T operand
    OT* sP = reinterpret_cast<OT*>(smem + C::R2);
    float* sBeta = reinterpret_cast<float*>(smem + C::R3);

    const int h = bx, s = by / a.Wc, jl = by % a.Wc;
    int64_t tb, L;
    seq_bounds(a, s, tb, L);
    const int64_t c0 = (int64_t)(a.win * a.Wc + jl) * CH;
    if (c0 >= L) return true;  // whole workgroup: no chunk here
    const int n = (int)min<int64_t>(CH, L - c0);
    const int64_t tok0 = tb + c0;
    const int H = a.H;

    const IT* q = static_cast<const IT*>(a.q);
    const IT* k = static_cast<const IT*>(a.k);
    const IT* v = static_cast<const IT*>(a.v);

    const int t = tid;
    // the wave index is uniform: held in a scalar register, loop bounds and tile
    // indices derived from it stay off the vector ALU
    const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int gq = lane >> 4, li = lane & 15;
    // this thread: channels ch, ch+1 over the 8 rows r0..r0+7 of half-block hb
    // (one half-block per wave when D = 128)
    constexpr int NP = D / 2;
    const int cp = t % NP, hb = NP == 64 ? wave : t / NP;
    const int ch = 2 * cp;
    const int b = hb >> 1, hh = hb & 1;  // 16-row block and which half of it
    const int r0 = 8 * hb;               // first row (within the chunk)
    const int ib0 = 8 * hh;              // first row within the block

    // ---- every global load first, in order of first use: gates, then k and q,
    // then v.  The barriers up to the off-diagonal operands order LDS only, so
    // k, q and v stay in flight while the gate products are formed.  Rows past
    // the end read the last valid row and are zeroed where first used.
    Pair8<IT> kraw, qraw, vv;
    float al[8][2];
    float bval;
    {
        // Raw gate words: an fp32 pair (log_alpha per channel) or one fp32 (per
        // head); with GPRE (the layer's gate pre-activation) a bf16 pair or one
        // bf16.  The branches only issue loads; the words are decoded after k, q
        // and v are in flight, so no branch waits for its own loads.
        uint32_t g0[8], g1[8];
        size_t off[8], th[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            th[i] = (size_t)(tok0 + min(r0 + i, n - 1)) * H + h;
            off[i] = th[i] * D + ch;
        }
        if constexpr (GPRE) {
            if (a.gate_per_head) {
#pragma unroll
                for (int i = 0; i < 8; ++i) g0[i] = a.gate[th[i]], g1[i] = 0u;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    g0[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.gate + off[i])), g1[i] = 0u;
            }
        } else {
            if (a.gate_per_head) {
#pragma unroll
                for (int i = 0; i < 8; ++i) g1[i] = g0[i] = __float_as_uint(a.la[th[i]]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    g0[i] = __float_as_uint(__builtin_nontemporal_load(a.la + off[i]));
                    g1[i] = __float_as_uint(__builtin_nontemporal_load(a.la + off[i] + 1));
                }
            }
        }
        // every thread loads a beta (no branch around a load); thread t < 64 stores row t
        bval = a.beta[(size_t)(tok0 + min(t & (CH - 1), n - 1)) * H + h];
#pragma unroll
        for (int i = 0; i < 8; ++i) kraw.load(i, k + off[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) qraw.load(i, q + off[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) vv.load(i, v + off[i]);
        if constexpr (GPRE) {  // bf16 gate pre-activation g: alpha = sigmoid(-g) = 1 / (1 + e^g)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x0 = __uint_as_float(g0[i] << 16);
                const float x1 = a.gate_per_head ? x0 : __uint_as_float(g0[i] & 0xFFFF0000u);
                al[i][0] = __builtin_amdgcn_rcpf(1.f + fast_exp(x0));
                al[i][1] = __builtin_amdgcn_rcpf(1.f + fast_exp(x1));
            }
        } else {  // log_alpha
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                al[i][0] = fast_exp(__uint_as_float(g0[i]));
                al[i][1] = fast_exp(__uint_as_float(g1[i]));
            }
        }
        // rows past the end decay by nothing (only in a sequence's last chunk; testing
        // n first keeps the gate loads out of any per-lane branch)
        if (n < CH) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (r0 + i >= n) al[i][0] = al[i][1] = 1.f;
        }
    }
    // half-block products, the half's first gate, and prod_{1..7} (first halves)
    float l7[2];  // this thread's prod_{1..7}, kept for the diagonal-block anchors
    {
        float hp[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            l7[e] = al[1][e];
#pragma unroll
            for (int i = 2; i < 8; ++i) l7[e] *= al[i][e];
            hp[e] = al[0][e] * l7[e];
        }
        *reinterpret_cast<float2*>(sX + hb * D + ch) = make_float2(hp[0], hp[1]);
        *reinterpret_cast<float2*>(sX + (8 + hb) * D + ch) = make_float2(al[0][0], al[0][1]);
        *reinterpret_cast<float2*>(sX + (16 + hb) * D + ch) = make_float2(l7[0], l7[1]);
    }
    if (t < CH) sBeta[t] = t < n ? bval : 0.f;
    // strictly-upper blocks of the staged P are zero (16 bytes per store)
    {
        constexpr int PER = 16 / sizeof(OT);
        for (int idx = t; idx < CH * CH / PER; idx += C::NT) {
            const int r = idx / (CH / PER), i = (idx % (CH / PER)) * PER;
            if ((i >> 4) > (r >> 4)) *reinterpret_cast<float4*>(sP + r * CH + i) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    lds_barrier();

    // per-channel products over blocks, half-blocks and anchors
    // (gam, the whole chunk's decay, and the record stores' starting factors Fs and Ks
    // are formed here, so the products they come from need not stay live to the end)
    float PB[4][2], A0[4][2], E[2], Sfx[2], HPo[2], HP0[2], L7[2], A8[2], gam[2], Fs[2], Ks[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            PB[x][e] = sX[(2 * x) * D + ch + e] * sX[(2 * x + 1) * D + ch + e];
            A0[x][e] = sX[(8 + 2 * x) * D + ch + e];
        }
        E[e] = 1.f;
        Sfx[e] = 1.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            if (x < b) E[e] *= PB[x][e];
            if (x > b) Sfx[e] *= PB[x][e];
        }
        gam[e] = ((PB[0][e] * PB[1][e]) * PB[2][e]) * PB[3][e];
        HPo[e] = sX[(2 * b + 1 - hh) * D + ch + e];  // the other half of this block
        HP0[e] = sX[(2 * b) * D + ch + e];           // the first half of this block
        L7[e] = sX[(16 + 2 * b) * D + ch + e];       // prod_{1..7} of the first half
        A8[e] = sX[(8 + 2 * b + 1) * D + ch + e];    // gate of the block's row 8
        // what the record stores need at the end: e^{G} of the row before this
        // thread's first, and e^{G_last - G} of its last row over the later rows
        Fs[e] = E[e] * (hh ? HP0[e] : 1.f);
        Ks[e] = Sfx[e] * (hh ? 1.f : HPo[e]);
    }
    const float* bb = sBeta + r0;  // beta of this thread's rows (LDS broadcast reads)
    lds_barrier();                 // sX is overwritten by the operands below
    typename QKReg<IT, QKN>::type kk, qq;
    if constexpr (QKN) {
        l2norm_rows<NP>(kraw, qraw, kk, qq, a.l2_eps);
    } else {
        kk = kraw;
        qq = qraw;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (r0 + i >= n) {
            kk.zero(i);
            qq.zero(i);
        }

    // ---- phase A: off-diagonal sub-blocks of Atil and P ----
    // rows 0..47  beta k e^{G_r - G_a}, blocks 1..3 (a = first row of the block)
    // rows 48..95 q e^{G_r - G_a}, blocks 1..3
    // rows 96..   k e^{G_a(rb) - G_i} for each (row block rb, column block cb < rb)
    if (b >= 1) {
        float Lf[2] = {hh ? L7[0] : 1.f, hh ? L7[1] : 1.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i > 0 || hh) {
                Lf[0] *= al[i][0];
                Lf[1] *= al[i][1];
            }
            const int row = 16 * (b - 1) + ib0 + i;
            put2<OT>(sOp + row * C::DP + ch, bb[i] * kk.get(i, 0) * Lf[0], bb[i] * kk.get(i, 1) * Lf[1]);
            put2<OT>(sOp + (48 + row) * C::DP + ch, qq.get(i, 0) * Lf[0], qq.get(i, 1) * Lf[1]);
        }
    }
    {
        float X[4][2];
#pragma unroll
        for (int rb = 1; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                X[rb][e] = A0[rb][e];  // e^{G_a(rb) - G_end(b)}
#pragma unroll
                for (int x = 1; x < 3; ++x)
                    if (x > b && x < rb) X[rb][e] *= PB[x][e];
            }
        float Rb[2] = {hh ? 1.f : HPo[0], hh ? 1.f : HPo[1]};  // e^{G_end(b) - G_row}
#pragma unroll
        for (int i = 7; i >= 0; --i) {
            if (i < 7) {
                Rb[0] *= al[i + 1][0];
                Rb[1] *= al[i + 1][1];
            }
#pragma unroll
            for (int rb = 1; rb < 4; ++rb)
                if (rb > b)
                    put2<OT>(sOp + (96 + 16 * (rb * (rb - 1) / 2 + b) + ib0 + i) * C::DP + ch,
                             kk.get(i, 0) * Rb[0] * X[rb][0], kk.get(i, 1) * Rb[1] * X[rb][1]);
        }
    }
    __syncthreads();
    for (int p = wave; p < 12; p += C::NW) {
        const int sl = p % 6;
        const int rb = sl == 0 ? 1 : (sl < 3 ? 2 : 3);
        const int cb = sl - rb * (rb - 1) / 2;
        floatx4 acc = zero4();
        mma_tile<OT>(acc, sOp + ((p < 6 ? 0 : 48) + 16 * (rb - 1)) * C::DP, C::DP, sOp + (96 + 16 * sl) * C::DP,
                     C::DP, D, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rb + 4 * gq + r, col = 16 * cb + li;
            if (p < 6)
                sAt[row * C::AP + col] = acc[r];
            else
                sP[row * CH + col] = from_f32<OT>(acc[r]);
        }
    }

    // ---- phase B: diagonal sub-blocks, anchored at row 8 of the block ----
    // rows 0..63 beta k e^{G_r - G_m}; 64..127 q e^{G_r - G_m}; 128..191 k e^{G_m - G_i}
    // With M_i = prod_{1..i} of this thread's gates (rows 8..15 of the block) or
    // B_i = a_8 prod_{i+1..7} (rows 0..7), the row factor dl_i is M_i or 1 / B_i and
    // the column factor dr_i is 1 / M_i or B_i.  Both follow from one reciprocal per
    // channel: dl_i = dl_{i-1} a_i forward from dl_0 = 1 or 1 / (a_8 prod_{1..7}),
    // dr_i = dr_{i+1} a_{i+1} backward from dr_7 = 1 / prod_{1..7} or a_8.
    float DL0[2], DR7[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float r = __builtin_amdgcn_rcpf(hh ? l7[e] : A8[e] * l7[e]);
        DL0[e] = hh ? 1.f : r;
        DR7[e] = hh ? r : A8[e];
    }
    auto dl_rows = [&](auto&& visit) {  // visit(i, dl_e0, dl_e1), i ascending
        float f[2] = {DL0[0], DL0[1]};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i > 0) {
                f[0] *= al[i][0];
                f[1] *= al[i][1];
            }
            visit(i, f[0], f[1]);
        }
    };
    auto dr_rows = [&](auto&& visit) {  // visit(i, dr_e0, dr_e1), i descending
        float f[2] = {DR7[0], DR7[1]};
#pragma unroll
        for (int i = 7; i >= 0; --i) {
            if (i < 7) {
                f[0] *= al[i + 1][0];
                f[1] *= al[i + 1][1];
            }
            visit(i, f[0], f[1]);
        }
    };
    const int rowB = 16 * b + ib0;  // first row of this thread in [0, 64)
    if constexpr (!WIDE) {
        // Range check of the single-anchor form: the largest row and column factors
        // (and, for fp16 operands, every operand's bound: the largest |k|, |q| and
        // |beta| over the thread's rows times those factors).  A zero gate can make a
        // factor infinite, and a later one in the same chain infinite times zero, but
        // the infinity comes first and already sets the maximum.
        int wide;
        {
            float km[2] = {0.f, 0.f}, qm[2] = {0.f, 0.f}, sb = 1.f, dlm[2] = {0.f, 0.f}, drm[2] = {0.f, 0.f};
            if (C::F16) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        km[e] = fmaxf(km[e], fabsf(kk.get(i, e)));
                        qm[e] = fmaxf(qm[e], fabsf(qq.get(i, e)));
                    }
                    sb = fmaxf(sb, fabsf(bb[i]));
                }
            }
            dl_rows([&](int, float f0, float f1) {
                dlm[0] = fmaxf(dlm[0], f0);
                dlm[1] = fmaxf(dlm[1], f1);
            });
            dr_rows([&](int, float f0, float f1) {
                drm[0] = fmaxf(drm[0], f0);
                drm[1] = fmaxf(drm[1], f1);
            });
            float mx = 0.f, fx = 0.f;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                mx = fmaxf(mx, fmaxf(fmaxf(km[e], qm[e]) * sb * dlm[e], km[e] * drm[e]));
                fx = fmaxf(fx, fmaxf(dlm[e], drm[e]));
            }
            wide = C::F16 ? __syncthreads_or(!(mx <= F16_OPERAND_LIMIT) || !(fx <= F16_FACTOR_LIMIT))
                          : __syncthreads_or(!(fx <= F32_FACTOR_LIMIT));
        }
        if (wide) return false;

        dl_rows([&](int i, float dl0, float dl1) {
            put2<OT>(sOp + (rowB + i) * C::DP + ch, bb[i] * kk.get(i, 0) * dl0, bb[i] * kk.get(i, 1) * dl1);
            put2<OT>(sOp + (64 + rowB + i) * C::DP + ch, qq.get(i, 0) * dl0, qq.get(i, 1) * dl1);
        });
        dr_rows([&](int i, float dr0, float dr1) {
            put2<OT>(sOp + (128 + rowB + i) * C::DP + ch, kk.get(i, 0) * dr0, kk.get(i, 1) * dr1);
        });
        __syncthreads();
        for (int p = wave; p < 8; p += C::NW) {
            const int db = p & 3;
            floatx4 acc = zero4();
            mma_tile<OT>(acc, sOp + ((p < 4 ? 0 : 64) + 16 * db) * C::DP, C::DP, sOp + (128 + 16 * db) * C::DP,
                         C::DP, D, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lr = 4 * gq + r;
                const int row = 16 * db + lr, col = 16 * db + li;
                if (p < 4)
                    sAt[row * C::AP + col] = acc[r];
                else
                    sP[row * CH + col] = from_f32<OT>(lr >= li ? acc[r] : 0.f);
            }
        }
        __syncthreads();
    } else {
        // Multi-level form (fp32 operands, two blocks at a time).  A pair (r, i),
        // i < r, of a diagonal block is formed at the level where r and i first
        // fall into different halves of an aligned sub-block of sz = 16, 8, 4, 2
        // rows.  The anchor is that sub-block's middle row m (the first row of its
        // later half): row r carries prod_{m < t <= r} alpha_t, column i carries
        // prod_{i < t <= m} alpha_t, both at most 1, so no gate is out of range.
        // Each level's product is kept only at its own pairs; the first level
        // also clears the rest of the block.  A last level (sz = 1) forms P's
        // diagonal, whose factor is 1.
#pragma unroll 1
        for (int lev = 0; lev < 5; ++lev) {
            const bool dg = lev == 4;
            const int sz = dg ? 1 : 16 >> lev, hs = sz >> 1, msk = sz - 1;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if ((b >> 1) == half) {
                    // Level 0 splits the block at its row 8: this thread's rows are the
                    // later half when hh = 1, the earlier half when hh = 0, and the earlier
                    // rows' anchor gate is that of the block's row 8 (another thread's row).
                    // Deeper levels split inside the thread's eight rows.
                    const int rr0 = 16 * (b & 1) + ib0;
                    float f0 = 1.f, f1 = 1.f;  // row factor, ascending
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const bool start = dg || (lev == 0 ? i == 0 : (i & msk) == hs);  // the anchor row
                        const bool later = dg || (lev == 0 ? hh == 1 : (i & msk) >= hs);
                        if (i > 0) {
                            f0 = start ? 1.f : f0 * al[i][0];
                            f1 = start ? 1.f : f1 * al[i][1];
                        }
                        const float m0 = later ? f0 : 0.f, m1 = later ? f1 : 0.f;
                        put2<float>(sOp32 + (rr0 + i) * C::DP32 + ch, bb[i] * kk.get(i, 0) * m0,
                                    bb[i] * kk.get(i, 1) * m1);
                        put2<float>(sOp32 + (32 + rr0 + i) * C::DP32 + ch, qq.get(i, 0) * m0, qq.get(i, 1) * m1);
                    }
                    float g0 = 1.f, g1 = 1.f;  // column factor, descending
#pragma unroll
                    for (int i = 7; i >= 0; --i) {
                        const bool last = lev == 0 ? i == 7 : (i & msk) == hs - 1;  // the row before the anchor
                        const bool earlier = lev == 0 ? hh == 0 : (i & msk) < hs;
                        // the gate of the block's row 8 is DR7 in the threads with hh = 0, the
                        // only ones whose level-0 column operands are kept
                        const float a0 = i == 7 ? DR7[0] : al[i < 7 ? i + 1 : 7][0];
                        const float a1 = i == 7 ? DR7[1] : al[i < 7 ? i + 1 : 7][1];
                        g0 = last ? a0 : g0 * a0;
                        g1 = last ? a1 : g1 * a1;
                        const float c0 = dg ? 1.f : (earlier ? g0 : 0.f), c1 = dg ? 1.f : (earlier ? g1 : 0.f);
                        put2<float>(sOp32 + (64 + rr0 + i) * C::DP32 + ch, kk.get(i, 0) * c0, kk.get(i, 1) * c1);
                    }
                }
                __syncthreads();
                for (int p = dg ? wave + 2 : wave; p < 4; p += C::NW) {  // the diagonal: P only
                    const int hbk = p & 1, db = 2 * half + hbk;
                    floatx4 acc = zero4();
                    // a short unroll: this rare path must not raise the kernel's register peak
                    const float* pa = sOp32 + ((p < 2 ? 0 : 32) + 16 * hbk + li) * C::DP32 + gq;
                    const float* pb = sOp32 + (64 + 16 * hbk + li) * C::DP32 + gq;
#pragma unroll 4
                    for (int k0 = 0; k0 < D; k0 += 4)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0], pb[k0], acc, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int lr = 4 * gq + r;
                        const bool pair = dg ? lr == li
                                             : (lr & ~msk) == (li & ~msk) && (lr & msk) >= hs && (li & msk) < hs;
                        const int row = 16 * db + lr, col = 16 * db + li;
                        if (pair || lev == 0) {
                            const float x = pair ? acc[r] : 0.f;
                            if (p < 2)
                                sAt[row * C::AP + col] = x;
                            else
                                sP[row * CH + col] = from_f32<OT>(x);
                        }
                    }
                }
                __syncthreads();
            }
        }
    }

    // ---- T = (I + Atil)^-1 (fp32) ----
    ut_inverse64<C::AP, C::NW>(sT, sAt, wave, lane);
    if (C::F16) {
        // eight consecutive columns of one row per step (16-byte stores)
        for (int idx = t; idx < CH * CH / 8; idx += C::NT) {
            const int r = idx / 8, i = (idx % 8) * 8;
            float x[8];
            const bool upper = (i >> 4) > (r >> 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = upper ? 0.f : sT[r * C::AP + i + e];
            store8<OT>(sTh + r * THP + i, x);
        }
    } else {
        for (int idx = t; idx < CH * CH; idx += C::NT) {
            const int r = idx / CH, i = idx % CH;
            if ((i >> 4) > (r >> 4)) sT[r * C::AP + i] = 0.f;
        }
    }
    __syncthreads();

    // ---- right-hand sides of W and Ut, channel-major: 8 tokens of each channel ----
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (r0 + i >= n) vv.zero(i);
    {
        float F[2] = {Fs[0], Fs[1]};  // e^{G} of the row before
        float x0[8], x1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            F[0] *= al[i][0];
            F[1] *= al[i][1];
            x0[i] = bb[i] * kk.get(i, 0) * F[0];
            x1[i] = bb[i] * kk.get(i, 1) * F[1];
        }
        store8<OT>(sKgT + (size_t)ch * C::KP + r0, x0);
        store8<OT>(sKgT + (size_t)(ch + 1) * C::KP + r0, x1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x0[i] = bb[i] * vv.get(i, 0);
            x1[i] = bb[i] * vv.get(i, 1);
        }
        store8<OT>(sVbT + (size_t)ch * C::KP + r0, x0);
        store8<OT>(sVbT + (size_t)(ch + 1) * C::KP + r0, x1);
    }
    __syncthreads();

    // ---- W = T (beta K e^G), Ut = T (beta V), then every record store ----
    unsigned char* rec = a.rec + ((size_t)(s * a.Wc + jl) * H + h) * a.rec_bytes;
    OT* rW = reinterpret_cast<OT*>(rec + R::W);
    OT* rQg = reinterpret_cast<OT*>(rec + R::QG);
    OT* rKhT = reinterpret_cast<OT*>(rec + R::KHT);
    OT* rP = reinterpret_cast<OT*>(rec + R::P);
    OT* rUt = reinterpret_cast<OT*>(rec + R::UT);
    float* rG = reinterpret_cast<float*>(rec + R::GAM);
    constexpr int NTC = D / 16;
    for (int p = wave; p < 8 * NTC; p += C::NW) {
        const bool isU = p >= 4 * NTC;
        const int rem = p % (4 * NTC);
        const int rb = rem / NTC, ct = rem % NTC;
        constexpr int KS = Mma<OT>::KSTEP;
        const int K = ((16 * (rb + 1) + KS - 1) / KS) * KS;
        floatx4 acc = zero4();
        if (isU) {
            // Ut tile: lane holds rows 16rb+4gq..+3 of value column 16ct+li
            mma_tile<OT>(acc, sTh + (16 * rb) * THP, THP, sVbT + (16 * ct) * C::KP, C::KP, K, lane);
            store4<OT>(rUt + ((size_t)rb * D + 16 * ct + li) * 16 + 4 * gq, acc);
        } else {
            // W^T = (beta K e^G)^T T^T: lane holds channels 16ct+4gq..+3 of row 16rb+li,
            // which are 4 consecutive elements in fragment order
            mma_tile<OT>(acc, sKgT + (16 * ct) * C::KP, C::KP, sTh + (16 * rb) * THP, THP, K, lane);
            if (C::F16) {
                store4<OT>(rW + FO::idx(16 * rb + li, 16 * ct + 4 * gq, D), acc);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) rW[FO::idx(16 * rb + li, 16 * ct + 4 * gq + e, D)] = from_f32<OT>(acc[e]);
            }
        }
    }
    {
        // Qg: the two channels of a row are adjacent in fragment order (ch is even)
        float F[2] = {Fs[0], Fs[1]};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            F[0] *= al[i][0];
            F[1] *= al[i][1];
            const int idx = FO::idx(r0 + i, ch, D);
            if (C::F16)
                put2<OT>(rQg + idx, qq.get(i, 0) * F[0], qq.get(i, 1) * F[1]);
            else {
                rQg[idx] = from_f32<OT>(qq.get(i, 0) * F[0]);
                rQg[FO::idx(r0 + i, ch + 1, D)] = from_f32<OT>(qq.get(i, 1) * F[1]);
            }
        }
        // Kh^T: 8 consecutive tokens of one channel are contiguous in fragment order (fp16)
        float x0[8], x1[8];
        float Rb[2] = {Ks[0], Ks[1]};  // e^{G_last - G_i}
#pragma unroll
        for (int i = 7; i >= 0; --i) {
            if (i < 7) {
                Rb[0] *= al[i + 1][0];
                Rb[1] *= al[i + 1][1];
            }
            x0[i] = kk.get(i, 0) * Rb[0];
            x1[i] = kk.get(i, 1) * Rb[1];
        }
        if (C::F16) {
            store8<OT>(rKhT + FO::idx(ch, r0, CH), x0);
            store8<OT>(rKhT + FO::idx(ch + 1, r0, CH), x1);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                rKhT[FO::idx(ch, r0 + i, CH)] = from_f32<OT>(x0[i]);
                rKhT[FO::idx(ch + 1, r0 + i, CH)] = from_f32<OT>(x1[i]);
            }
        }
        if (hb == 0)
            *reinterpret_cast<float2*>(rG + ch) =
                make_float2(gam[0], gam[1]);
    }
    for (int f = t; f < CH * CH / FO::KE; f += C::NT) {  // P: one lane slot of one fragment per step
        const int l = f & 63, kk2 = (f >> 6) % (CH / FO::KS), rt = (f >> 6) / (CH / FO::KS);
        const OT* src = sP + (16 * rt + (l & 15)) * CH + kk2 * FO::KS + (l >> 4) * FO::KE;
        OT* dst = rP + (size_t)f * FO::KE;
        if (FO::KE == 8)
            *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
        else
            dst[0] = src[0];
    }
    return true;
}

// A chunk whose single-anchor factors leave their range is marked in its
// record with an impossible decay (gamma[0] = -1) and formed by the next kernel.
constexpr float WIDE_MARK = -1.f;

template <int D, typename IT, typename OT, bool QKN, bool GPRE>
__global__ void __launch_bounds__(4 * D) __attribute__((amdgpu_waves_per_eu(4))) chunk_local_kernel(ChunkArgs a) {
    __shared__ __align__(16) unsigned char smem[LocalCfg<D, OT>::SMEM];
    if (!chunk_local_body<D, IT, OT, QKN, GPRE, false>(a, smem, blockIdx.x, blockIdx.y, threadIdx.x) &&
        threadIdx.x == 0) {
        const int s = blockIdx.y / a.Wc, jl = blockIdx.y % a.Wc;
        unsigned char* rec = a.rec + ((size_t)(s * a.Wc + jl) * a.H + blockIdx.x) * a.rec_bytes;
        reinterpret_cast<float*>(rec + Rec<D, OT>::GAM)[0] = WIDE_MARK;
    }
}

// The chunks chunk_local_kernel declined, in the multi-level form.  A kernel of
// its own, so the common form keeps its registers.  Workgroup w takes a
// contiguous range of at most 4 D (its thread count) chunk slots of the window,
// slot = (sequence, chunk in window, head); every thread reads one slot's mark,
// and the workgroup then forms the marked chunks one after another.
template <int D, typename IT, typename OT, bool QKN, bool GPRE>
__global__ void __launch_bounds__(4 * D) chunk_local_wide_kernel(ChunkArgs a, int per_wg) {
    constexpr int NT = 4 * D;
    __shared__ __align__(16) unsigned char smem[LocalCfg<D, OT>::SMEM];
    __shared__ int marked[NT];
    __shared__ int nmarked;
    const int t = threadIdx.x;
    const int64_t slots = (int64_t)a.N * a.Wc * a.H;
    const int64_t first = (int64_t)blockIdx.x * per_wg;
    if (t == 0) nmarked = 0;
    __syncthreads();
    if (t < per_wg && first + t < slots) {
        const int64_t slot = first + t;
        const int h = (int)(slot % a.H), y = (int)(slot / a.H);  // y = s * Wc + jl
        const int s = y / a.Wc, jl = y % a.Wc;
        int64_t tb, L;
        seq_bounds(a, s, tb, L);
        // a slot past its sequence's end was not written this window: not a chunk
        if ((int64_t)(a.win * a.Wc + jl) * CH < L) {
            const unsigned char* rec = a.rec + (size_t)slot * a.rec_bytes;
            if (reinterpret_cast<const float*>(rec + Rec<D, OT>::GAM)[0] == WIDE_MARK)
                marked[atomicAdd(&nmarked, 1)] = (int)(slot - first);
        }
    }
    __syncthreads();
    const int n = nmarked;
    for (int i = 0; i < n; ++i) {
        const int64_t slot = first + marked[i];
        chunk_local_body<D, IT, OT, QKN, GPRE, true>(a, smem, (int)(slot % a.H), (int)(slot / a.H), t);
        __syncthreads();  // smem is reused by the next marked chunk
    }
}

// Both chunk-local kernels over one window (or every chunk).
template <int D, typename IT, typename OT, bool QKN, bool GPRE>
static hipError_t launch_local(const ChunkArgs& a, hipStream_t st) {
    using C = LocalCfg<D, OT>;
    hipLaunchKernelGGL((chunk_local_kernel<D, IT, OT, QKN, GPRE>), dim3(a.H, a.N * a.Wc), dim3(C::NT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // at most 256 workgroups (one per compute unit), each over a contiguous range of slots
    const int64_t slots = (int64_t)a.N * a.Wc * a.H;
    const int per_wg = (int)std::min<int64_t>(C::NT, std::max<int64_t>(1, (slots + 255) / 256));
    const int64_t wgs = (slots + per_wg - 1) / per_wg;
    hipLaunchKernelGGL((chunk_local_wide_kernel<D, IT, OT, QKN, GPRE>), dim3((unsigned)wgs), dim3(C::NT), 0, st, a,
                       per_wg);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// inter-chunk kernel
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per (sequence, head, slice of BV value columns).
// Waves 0..3 carry the state: for chunk j they form U_j = Ut_j - W_j S_j and
// S_{j+1} = Diag(gamma_j) S_j + Kh_j^T U_j, the only dependent chain.  Waves
// 4..7 form the outputs O_j = Qg_j S_j + P_j U_j off that chain.  S_j and U_j
// pass between the two groups through double-buffered fp16 LDS tiles; two
// barriers per chunk.  Each wave keeps the record fragments it needs for the
// next RING-1 chunks in registers (a ring of RING buffers).
//
// A chunk step moves about 57 KB of record through the CU's vector memory
// path, which is the step's real cost, so the loads are spread over the two
// phases of the step: the output waves and the chain's Kh^T loads are issued
// right after the first barrier (while the chain computes U_j), the chain's
// W, Ut and gamma loads after its state update.  Prefetches are unconditional
// (the chunk index is clamped to the window, so past the end the last record
// is read again) except the chain's Kh^T, which is only needed by steps that
// run; this keeps the compiler's load-count waits exact.
// MODE 0: one window of chunks, state carried in state_buf between windows.
// MODE 1 (sequence-parallel, first pass): workgroup (unit, slice, segment g)
//   runs segment g's chunks from a zero state and writes the end state to
//   seg_B; slices D/BV .. 2D/BV-1 instead carry the dk columns of the
//   segment's transition product, starting from the identity with Ut = 0
//   (each column obeys S <- (Diag(gamma) - Kh^T W) S), written to seg_M.  No
//   outputs.
// MODE 2 (second pass): each segment from its true initial state (seg_init),
//   forming the outputs; the final state is written by the combine kernel.
// SNAP (with MODE 0, no outputs): the chain waves leave the fp32 state entering
//   each chunk in LDS and the output waves store it to a.snap, off the chain.
template <int D, int BV, typename OT, typename OUT, int MODE = 0, bool SNAP = false>
__global__ void __launch_bounds__(512) chunk_inter_kernel(ChunkArgs a) {
    using R = Rec<D, OT>;
    using FR = Frag<OT>;
    using FT = typename FR::T;
    constexpr int KS = Mma<OT>::KSTEP;
    constexpr int NFD = D / KS;   // fragments along a D-long row
    constexpr int NFT = CH / KS;  // fragments along a 64-long row
    constexpr int RT = D / 64;    // 16-row state tiles per chain wave
    constexpr int CT = BV / 16;   // 16-column tiles
    constexpr int PD = Pad<OT>::v;
    constexpr int SP = D + PD;
    constexpr int UP = CH + PD;
    constexpr int RING = sizeof(OT) == 2 ? (BV <= 32 ? 3 : 2) : 1;
    __shared__ __align__(16) OT sS[2][BV * SP];
    __shared__ __align__(16) OT sU[2][BV * UP];
    constexpr int SNP = BV + 1;
    __shared__ float sSnap[SNAP ? D * SNP : 1];
    __shared__ float sUsnap[SNAP ? CH * SNP : 1];

    constexpr int ZS = D / BV;                   // slices of the value columns
    constexpr int Z = MODE == 1 ? 2 * ZS : ZS;  // the first segment pass also carries the transition product
    const int H = a.H;
    const int NH = a.N * H;
    const int u = blockIdx.x % NH, z = (blockIdx.x / NH) % Z;
    const int seg = MODE == 0 ? 0 : (int)(blockIdx.x / NH) / Z;
    const bool mslice = MODE == 1 && z >= ZS;   // a slice of the transition product
    const int s = u / H, h = u % H;
    int64_t tb, L;
    seq_bounds(a, s, tb, L);
    const int nchunks = (int)((L + CH - 1) / CH);
    const int jb = MODE == 0 ? a.win * a.Wc : seg * a.Sc;
    // the segment passes hold a record for each of the first Wc chunks only: a
    // sequence longer than the launch was sized for is truncated there, as the
    // windowed pass (whose chunk index never leaves its window) truncates it
    const int je = min(MODE == 0 ? nchunks : min(nchunks, a.Wc), MODE == 0 ? jb + a.Wc : jb + a.Sc);
    if (MODE == 0 ? (jb >= je && a.win > 0) : jb >= je) return;
    const int jrec0 = MODE == 0 ? jb : 0;        // first chunk held by the record buffer

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const bool chain = wave < 4;
    const int w = wave & 3;
    const int gq = lane >> 4, li = lane & 15;
    const int col0 = (mslice ? z - ZS : z) * BV;
    OUT* out = static_cast<OUT*>(a.out);

    auto rec_of = [&](int j) {
        return a.rec + ((size_t)(s * a.Wc + (j - jrec0)) * H + h) * a.rec_bytes;
    };
    floatx4 Sacc[RT][CT];
    if (chain) {
        const float* src;
        if (MODE == 0) {
            src = a.win == 0 ? a.init : a.state_buf;
            if (src) src += (size_t)u * D * D;
        } else if (MODE == 1) {
            src = nullptr;  // zero state, or the identity for the transition product
        } else {
            src = a.seg_init + ((size_t)u * a.G + seg) * D * D;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = w * (D / 4) + 16 * rt + 4 * gq + r;
                    const int col = col0 + 16 * ct + li;
                    Sacc[rt][ct][r] = src ? src[(size_t)row * D + col] : (mslice && row == col ? 1.f : 0.f);
                }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                store4<OT>(&sS[0][(16 * ct + li) * SP + w * (D / 4) + 16 * rt + 4 * gq], Sacc[rt][ct]);

        // state chain: W, Kh^T, Ut and gamma of one chunk
        struct ChainBuf {
            FT W[NFD];
            FT K[RT][NFT];
            floatx4 U[CT];
            float G;  // gamma of state row w*D/4 + lane % (D/4)
        };
        auto load = [&](ChainBuf& f, int j) {
            const unsigned char* rec = rec_of(j);
            using FO = FragOrder<OT>;
            const OT* rW = reinterpret_cast<const OT*>(rec + R::W);
#pragma unroll
            for (int e = 0; e < NFD; ++e) f.W[e] = FR::load(rW + FO::frag(w, e, lane, D), 0);
            // one dword per lane (a 16-byte load per lane would move 16x the bytes gamma has)
            f.G = reinterpret_cast<const float*>(rec + R::GAM)[w * (D / 4) + lane % (D / 4)];
            const OT* rUt = reinterpret_cast<const OT*>(rec + R::UT);
            // the transition product sees Ut = 0 (scaled, so the load stays unconditional)
            const float umask = mslice ? 0.f : 1.f;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f.U[ct] = load4<OT>(rUt + ((size_t)w * D + col0 + 16 * ct + li) * 16 + 4 * gq);
#pragma unroll
                for (int r = 0; r < 4; ++r) f.U[ct][r] *= umask;
            }
        };
        auto loadK = [&](ChainBuf& f, int j) {
            using FO = FragOrder<OT>;
            const OT* rK = reinterpret_cast<const OT*>(rec_of(j) + R::KHT);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int e = 0; e < NFT; ++e) f.K[rt][e] = FR::load(rK + FO::frag(w * RT + rt, e, lane, CH), 0);
        };
        auto step = [&](ChainBuf& f, ChainBuf& fn, int jn, int j) {
            const int cur = (j - jb) & 1;
            if constexpr (SNAP) {  // the state entering chunk j, for the backward pass
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            sSnap[(w * (D / 4) + 16 * rt + 4 * gq + r) * SNP + 16 * ct + li] = Sacc[rt][ct][r];
            }
            float g[RT][4];  // gamma of the four state rows each accumulator lane holds
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) g[rt][r] = __shfl(f.G, 16 * rt + 4 * gq + r);
            lds_barrier();  // S_j is in sS[cur]
            loadK(fn, jn);  // Kh^T of a later chunk, issued in the phase where the output waves compute
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                floatx4 acc = zero4();
                const OT* bt = sS[cur] + (16 * ct + li) * SP;
#pragma unroll
                for (int e = 0; e < NFD; ++e) acc = FR::mma(f.W[e], bt + e * KS, gq, acc);
                floatx4 Uv;
#pragma unroll
                for (int r = 0; r < 4; ++r) Uv[r] = f.U[ct][r] - acc[r];
                store4<OT>(sU[cur] + (16 * ct + li) * UP + 16 * w + 4 * gq, Uv);
                if constexpr (SNAP) {  // U_j in fp32, for the backward pass
#pragma unroll
                    for (int r = 0; r < 4; ++r) sUsnap[(16 * w + 4 * gq + r) * SNP + 16 * ct + li] = Uv[r];
                }
            }
            lds_barrier();  // U_j is in sU[cur]
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sacc[rt][ct][r] *= g[rt][r];
                    const OT* bt = sU[cur] + (16 * ct + li) * UP;
#pragma unroll
                    for (int e = 0; e < NFT; ++e) Sacc[rt][ct] = FR::mma(f.K[rt][e], bt + e * KS, gq, Sacc[rt][ct]);
                }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    store4<OT>(sS[cur ^ 1] + (16 * ct + li) * SP + w * (D / 4) + 16 * rt + 4 * gq, Sacc[rt][ct]);
        };
        ChainBuf buf[RING];
        if (jb < je) {
#pragma unroll
            for (int p = 0; p + 1 < RING; ++p) {
                load(buf[p], min(jb + p, je - 1));
                loadK(buf[p], min(jb + p, je - 1));
            }
            for (int j0 = jb; j0 < je; j0 += RING) {
#pragma unroll
                for (int p = 0; p < RING; ++p) {
                    const int j = j0 + p, jn = min(j + RING - 1, je - 1);
                    load(buf[(p + RING - 1) % RING], jn);
                    if (j < je) step(buf[p], buf[(p + RING - 1) % RING], jn, j);
                }
            }
        }
    } else if constexpr (SNAP) {
        // no outputs: between the step's two barriers, store the chain's fp32 copy of
        // S_j; after the second, U_j (the chain writes the next U only after the next
        // step's first barrier)
        for (int j = jb; j < je; ++j) {
            lds_barrier();  // S_j is in sSnap
            const size_t chh = (size_t)(s * a.snap_wc + (j - a.snap_j0)) * H + h;
            float* dst = a.snap + chh * D * D + col0;
            for (int idx = t - 256; idx < D * BV / 4; idx += 256) {  // 16 bytes per lane
                const int k = idx / (BV / 4), c = 4 * (idx % (BV / 4));
                const float* sp = sSnap + k * SNP + c;
                *reinterpret_cast<float4*>(dst + (size_t)k * D + c) = make_float4(sp[0], sp[1], sp[2], sp[3]);
            }
            lds_barrier();  // U_j is in sUsnap
            if (a.snapU) {
                float* du = a.snapU + chh * a.snapU_stride + col0;
                for (int idx = t - 256; idx < CH * BV / 4; idx += 256) {
                    const int r = idx / (BV / 4), c = 4 * (idx % (BV / 4));
                    const float* sp = sUsnap + r * SNP + c;
                    *reinterpret_cast<float4*>(du + (size_t)r * D + c) = make_float4(sp[0], sp[1], sp[2], sp[3]);
                }
            }
        }
    } else if constexpr (MODE == 1) {
        for (int j = jb; j < je; ++j) {  // no outputs in this pass; keep the barrier count
            lds_barrier();
            lds_barrier();
        }
    } else {
        // outputs: Qg and P of one chunk
        struct OutBuf {
            FT Q[NFD];
            FT P[NFT];
        };
        auto load = [&](OutBuf& f, int j) {
            const unsigned char* rec = rec_of(j);
            using FO = FragOrder<OT>;
            const OT* rQ = reinterpret_cast<const OT*>(rec + R::QG);
#pragma unroll
            for (int e = 0; e < NFD; ++e) f.Q[e] = FR::load(rQ + FO::frag(w, e, lane, D), 0);
            const OT* rP = reinterpret_cast<const OT*>(rec + R::P);
#pragma unroll
            for (int e = 0; e < NFT; ++e) f.P[e] = FR::load(rP + FO::frag(w, e, lane, CH), 0);
        };
        // called after the first barrier of chunk j (S_j is in sS[cur])
        auto step = [&](OutBuf& f, int j) {
            const int cur = (j - jb) & 1;
            floatx4 accO[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                floatx4 acc = zero4();
                const OT* bt = sS[cur] + (16 * ct + li) * SP;
#pragma unroll
                for (int e = 0; e < NFD; ++e) acc = FR::mma(f.Q[e], bt + e * KS, gq, acc);
                accO[ct] = acc;
            }
            lds_barrier();  // U_j is in sU[cur]
            const int n = (int)min<int64_t>(CH, L - (int64_t)j * CH);
            const int64_t tok0 = tb + (int64_t)j * CH;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const OT* bt = sU[cur] + (16 * ct + li) * UP;
#pragma unroll
                for (int e = 0; e < NFT; ++e) accO[ct] = FR::mma(f.P[e], bt + e * KS, gq, accO[ct]);
                if (!out) continue;  // state snapshots only
                OUT* o = out + ((size_t)(tok0 + 16 * w + 4 * gq) * H + h) * D + col0 + 16 * ct + li;
                if (n == CH) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) store_out(o + (size_t)r * H * D, accO[ct][r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * w + 4 * gq + r < n) store_out(o + (size_t)r * H * D, accO[ct][r]);
                }
            }
        };
        // The output waves issue their record loads right after the first
        // barrier, while the chain waves compute U_j from LDS and registers, so
        // the loads do not queue behind the chain's own at the end of the step.
        OutBuf buf[RING];
        if (jb < je) {
#pragma unroll
            for (int p = 0; p + 1 < RING; ++p) load(buf[p], min(jb + p, je - 1));
            for (int j0 = jb; j0 < je; j0 += RING) {
#pragma unroll
                for (int p = 0; p < RING; ++p) {
                    const int j = j0 + p;
                    if (j < je) lds_barrier();  // S_j is in sS[cur]
                    load(buf[(p + RING - 1) % RING], min(j + RING - 1, je - 1));
                    if (j < je) step(buf[p], j);
                }
            }
        }
    }

    if (chain && MODE != 2) {
        float* dst = MODE == 0 ? a.state_buf + (size_t)u * D * D
                               : (mslice ? a.seg_M : a.seg_B) + ((size_t)u * a.G + seg) * D * D;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = w * (D / 4) + 16 * rt + 4 * gq + r;
                    dst[(size_t)row * D + col0 + 16 * ct + li] = Sacc[rt][ct][r];
                }
    }
}

// Sequence-parallel state pass, combine step: one workgroup per (unit, 16
// value columns).  S_0 is the initial state (or 0); for each segment g,
// seg_init[g] = S_g and, if the segment holds chunks, S_{g+1} = M_g S_g + B_g
// (fp32).  The final state S_G goes to state_buf.
template <int D>
__global__ void __launch_bounds__(256) chunk_segment_combine_kernel(ChunkArgs a) {
    constexpr int TPR = 256 / D;    // threads per state row
    constexpr int CPT = 16 / TPR;   // columns per thread
    __shared__ float sS[D][16];
    const int u = blockIdx.x, c0 = 16 * blockIdx.y;
    const int t = threadIdx.x, row = t / TPR, cb = (t % TPR) * CPT;
    int64_t tb, L;
    seq_bounds(a, u / a.H, tb, L);
    const int nchunks = (int)((L + CH - 1) / CH);
    float x[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) x[c] = a.init ? a.init[((size_t)u * D + row) * D + c0 + cb + c] : 0.f;
    for (int g = 0; g < a.G; ++g) {
        const size_t blk = ((size_t)u * a.G + g) * D * D;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            a.seg_init[blk + (size_t)row * D + c0 + cb + c] = x[c];
            sS[row][cb + c] = x[c];
        }
        __syncthreads();
        if (g * a.Sc < min(nchunks, a.Wc)) {  // uniform; segments past the records hold no chunk
            float y[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) y[c] = a.seg_B[blk + (size_t)row * D + c0 + cb + c];
            const float* Mr = a.seg_M + blk + (size_t)row * D;
            for (int k = 0; k < D; ++k) {
                const float m = Mr[k];
#pragma unroll
                for (int c = 0; c < CPT; ++c) y[c] += m * sS[k][cb + c];
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) x[c] = y[c];
        }
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) a.state_buf[((size_t)u * D + row) * D + c0 + cb + c] = x[c];
}

// ---------------------------------------------------------------------------
// layer epilogue
// ---------------------------------------------------------------------------
// Head-wise RMSNorm and sigmoid output gate ("Kimi Delta Attention" section):
// y = o / sqrt(mean_j o_j^2 + eps) * w * sigmoid(z) per (token, head), in place
// in `out` over chunks win * Wc .. win * Wc + Wc - 1 of every sequence.  o is what the state pass wrote (OI:
// fp16 when y is bf16, else fp32); the mean needs a row's dv values, which the
// state pass spreads over its value-slice workgroups, hence a pass of its own.
// One workgroup per (head, chunk); LPR lanes hold a row, eight values each.
template <int D, typename OI>
__global__ void __launch_bounds__(256) layer_epilogue_kernel(ChunkArgs a) {
    using OF = typename std::conditional<std::is_same<OI, float>::value, float, bf16_t>::type;
    constexpr int LPR = D / 8, RPP = 256 / LPR;
    const int h = blockIdx.x, s = blockIdx.y / a.Wc, jl = blockIdx.y % a.Wc;
    int64_t tb, L;
    seq_bounds(a, s, tb, L);
    const int64_t c0 = (int64_t)(a.win * a.Wc + jl) * CH;
    if (c0 >= L) return;
    const int n = (int)min<int64_t>(CH, L - c0);
    const int t = threadIdx.x, lr = t / LPR, j0 = 8 * (t % LPR);
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = a.norm_weight ? a.norm_weight[j0 + e] : 1.f;
    // every row's o and z are loaded before any row is reduced (rows past the end
    // read the chunk's last row and are not stored)
    constexpr int NR = CH / RPP;  // rows per thread
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    float ov[NR][8];
    u32x4 zv[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const size_t base = ((size_t)(tb + c0 + min(lr + RPP * i, n - 1)) * a.H + h) * D + j0;
        if constexpr (std::is_same<OI, float>::value) {
            const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.out) + base);
            const float4 x0 = src[0], x1 = src[1];
            ov[i][0] = x0.x; ov[i][1] = x0.y; ov[i][2] = x0.z; ov[i][3] = x0.w;
            ov[i][4] = x1.x; ov[i][5] = x1.y; ov[i][6] = x1.z; ov[i][7] = x1.w;
        } else {
            const half8 x = *reinterpret_cast<const half8*>(static_cast<const _Float16*>(a.out) + base);
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[i][e] = (float)x[e];
        }
        zv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.out_gate + base));
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int r = lr + RPP * i;  // uniform over the LPR lanes of a row
        const size_t base = ((size_t)(tb + c0 + min(r, n - 1)) * a.H + h) * D + j0;
        const float* o = ov[i];
        float y[8];
        const uint32_t zw[4] = {zv[i][0], zv[i][1], zv[i][2], zv[i][3]};
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += o[e] * o[e];
#pragma unroll
        for (int off = 1; off < LPR; off *= 2) ss += __shfl_xor(ss, off);
        const float rs = __builtin_amdgcn_rsqf(ss * (1.f / D) + a.rms_eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t zw2 = zw[e >> 1];
            const float z = __uint_as_float((e & 1) ? (zw2 & 0xFFFF0000u) : (zw2 << 16));
            y[e] = o[e] * rs * w[e] * __builtin_amdgcn_rcpf(1.f + fast_exp(-z));
        }
        if (r >= n) continue;
        OF* dst = static_cast<OF*>(a.out) + base;
        if constexpr (std::is_same<OF, float>::value) {
            const floatx4 y0 = {y[0], y[1], y[2], y[3]}, y1 = {y[4], y[5], y[6], y[7]};
            __builtin_nontemporal_store(y0, reinterpret_cast<floatx4*>(dst));
            __builtin_nontemporal_store(y1, reinterpret_cast<floatx4*>(dst) + 1);
        } else {
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pk[e] = uint32_t(f32_to_bf16(y[2 * e]).bits) | (uint32_t(f32_to_bf16(y[2 * e + 1]).bits) << 16);
            typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
            const u32x4s pv = {pk[0], pk[1], pk[2], pk[3]};
            __builtin_nontemporal_store(pv, reinterpret_cast<u32x4s*>(dst));
        }
    }
}

template <int D, typename OUT>
static hipError_t launch_epilogue(const ChunkArgs& a, hipStream_t st) {
    if constexpr (std::is_same<OUT, bf16_t>::value) {
        return hipErrorInvalidValue;  // the state pass writes fp16 or fp32 when an epilogue follows
    } else {
        if (!a.out_gate) return hipSuccess;
        hipLaunchKernelGGL((layer_epilogue_kernel<D, OUT>), dim3(a.H, a.N * a.Wc), dim3(256), 0, st, a);
        return hipGetLastError();
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
size_t chunk_record_bytes(int d, bool in_bf16) {
    if (d == 128) return in_bf16 ? Rec<128, _Float16>::BYTES : Rec<128, float>::BYTES;
    return in_bf16 ? Rec<64, _Float16>::BYTES : Rec<64, float>::BYTES;
}

// Value-column slice of the sequence-parallel state pass.
constexpr int SEGMENT_BV = 16;

// Width of the value-column slice each state workgroup carries.  Narrow slices
// give more workgroups when there are few (sequence, head) pairs; wide ones
// read each chunk record fewer times.  KDA_VALUE_SLICE (16, 32 or 64) overrides.
int chunk_value_slice(int d, int64_t units) {
    const char* e = getenv("KDA_VALUE_SLICE");  // read per call
    const int v = e ? atoi(e) : 0;
    const int forced = (v == 16 || v == 32 || v == 64) ? v : 0;
    if (forced) return forced > d ? d : forced;
    if (units <= 64) return 16;
    if (units <= 256 || d == 64) return 32;
    return 64;
}

// Window loop: per window of chunks, the chunk-local pass then the state pass,
// both on the caller's stream; the records of one window live in the
// workspace between the two.
template <int D, typename IT, typename OT, typename OUT, bool QKN, bool GPRE, int BV>
static hipError_t run_windows(const ChunkArgs& base, int nwin, hipStream_t st) {
    using C = LocalCfg<D, OT>;
    const int units = base.N * base.H;
    for (int w = 0; w < nwin; ++w) {
        ChunkArgs a = base;
        a.win = w;
        hipError_t e;
        if ((e = launch_local<D, IT, OT, QKN, GPRE>(a, st)) != hipSuccess) return e;
        hipLaunchKernelGGL((chunk_inter_kernel<D, BV, OT, OUT>), dim3(units * (D / BV)), dim3(512), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!base.out_gate) return hipSuccess;
    // the epilogue after the last state pass (between state passes it would
    // evict the records they read): one launch over every window's chunks when
    // its grid rows (sequences x chunks) fit, else window by window
    if ((int64_t)base.N * nwin * base.Wc <= 65535) {
        ChunkArgs a = base;
        a.win = 0;
        a.Wc = nwin * base.Wc;
        return launch_epilogue<D, OUT>(a, st);
    }
    for (int w = 0; w < nwin; ++w) {
        ChunkArgs a = base;
        a.win = w;
        hipError_t e = launch_epilogue<D, OUT>(a, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Sequence-parallel state pass: all records in one buffer (a.win = 0, a.Wc =
// every chunk), a.G segments of a.Sc chunks per sequence.
template <int D, typename IT, typename OT, typename OUT, bool QKN, bool GPRE>
static hipError_t run_segments(const ChunkArgs& a, hipStream_t st) {
    using C = LocalCfg<D, OT>;
    constexpr int BV = SEGMENT_BV;
    const int NH = a.N * a.H;
    hipError_t e;
    if ((e = launch_local<D, IT, OT, QKN, GPRE>(a, st)) != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_inter_kernel<D, BV, OT, OUT, 1>), dim3(NH * 2 * (D / BV) * a.G), dim3(512), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_segment_combine_kernel<D>), dim3(NH, D / 16), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_inter_kernel<D, BV, OT, OUT, 2>), dim3(NH * (D / BV) * a.G), dim3(512), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return a.out_gate ? launch_epilogue<D, OUT>(a, st) : hipSuccess;
}

int chunk_segments(int d, int bv, int64_t units, int64_t max_chunks, int& chunks_per_segment) {
    chunks_per_segment = 0;
    if (bv != SEGMENT_BV || max_chunks < 2) return 0;
    const char* e = getenv("KDA_SEGMENTS");  // read per call: "0" turns the sequence-parallel pass off
    int64_t G;
    if (e && e[0] >= '0' && e[0] <= '9') {
        G = atoi(e);
    } else {
        // Measured on MI355X at 64K tokens: with at most 32 state-pass workgroups
        // (4 heads of one sequence) the split pays, best at 128-256 workgroups in
        // the second pass and no more than 16 segments; at 64 it no longer does.
        const int64_t wgs = units * (d / bv);  // state-pass workgroups of the windowed schedule
        if (wgs > 32 || max_chunks < 32) return 0;
        G = std::min<int64_t>(std::min<int64_t>(16, 256 / wgs), max_chunks / 16);
    }
    G = std::min<int64_t>(G, max_chunks);
    if (G < 2) return 0;
    const int64_t sc = (max_chunks + G - 1) / G;
    chunks_per_segment = (int)sc;
    return (int)((max_chunks + sc - 1) / sc);
}

template <int D, typename IT, typename OT, typename OUT, bool QKN, bool GPRE>
static hipError_t run_bv(const ChunkArgs& a, int nwin, int bv, hipStream_t st) {
    if (a.G > 0) return run_segments<D, IT, OT, OUT, QKN, GPRE>(a, st);
    if (bv == 16) return run_windows<D, IT, OT, OUT, QKN, GPRE, 16>(a, nwin, st);
    if (bv == 32) return run_windows<D, IT, OT, OUT, QKN, GPRE, 32>(a, nwin, st);
    return run_windows<D, IT, OT, OUT, QKN, GPRE, 64>(a, nwin, st);
}

// Output type of the state pass: the result's type, or fp16 in place of bf16
// when the layer epilogue follows (it reads o back and writes bf16 over it).
template <int D, typename IT, typename OT, bool QKN, bool GPRE>
static hipError_t run_out(const ChunkArgs& a, bool out_bf16, int nwin, int bv, hipStream_t st) {
    if (!out_bf16) return run_bv<D, IT, OT, float, QKN, GPRE>(a, nwin, bv, st);
    if (a.out_gate) return run_bv<D, IT, OT, _Float16, QKN, GPRE>(a, nwin, bv, st);
    return run_bv<D, IT, OT, bf16_t, QKN, GPRE>(a, nwin, bv, st);
}

// The plain operator (log_alpha, q and k as given) or the layer (gate
// pre-activation, q and k normalised or not).
template <int D, typename IT, typename OT>
static hipError_t run_norm(const ChunkArgs& a, bool out_bf16, bool qk_norm, int nwin, int bv, hipStream_t st) {
    if (!a.gate) return run_out<D, IT, OT, false, false>(a, out_bf16, nwin, bv, st);
    if (qk_norm) return run_out<D, IT, OT, true, true>(a, out_bf16, nwin, bv, st);
    return run_out<D, IT, OT, false, true>(a, out_bf16, nwin, bv, st);
}

// Record windows w0 .. w0 + nw - 1 of `window` chunks: the records of one
// window stay in the last-level cache between its two passes, and the state
// pass carries S through state_buf.  With SNAP the state pass stores the state
// entering every chunk; without it, it only carries S (no outputs either).
template <int D, typename IT, typename OT>
static hipError_t run_snapshots(const ChunkArgs& base, int window, int w0, int nw, bool snap, hipStream_t st) {
    using C = LocalCfg<D, OT>;
    for (int w = w0; w < w0 + nw; ++w) {
        ChunkArgs a = base;
        a.Wc = window;
        a.win = w;
        a.out = nullptr;
        hipError_t e = launch_local<D, IT, OT, false, false>(a, st);
        if (e != hipSuccess) return e;
        if (snap)
            hipLaunchKernelGGL((chunk_inter_kernel<D, 16, OT, float, 0, true>), dim3(a.N * a.H * (D / 16)), dim3(512),
                               0, st, a);
        else
            hipLaunchKernelGGL((chunk_inter_kernel<D, 16, OT, float, 0, false>), dim3(a.N * a.H * (D / 16)),
                               dim3(512), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t chunk_snapshot_dispatch(int d, bool in_bf16, const ChunkArgs& a, int window, int w0, int nw, bool snap,
                                   hipStream_t st, bool f32_operands) {
    if (d == 128) {
        if (in_bf16 && f32_operands) return run_snapshots<128, bf16_t, float>(a, window, w0, nw, snap, st);
        return in_bf16 ? run_snapshots<128, bf16_t, _Float16>(a, window, w0, nw, snap, st)
                       : run_snapshots<128, float, float>(a, window, w0, nw, snap, st);
    }
    if (in_bf16 && f32_operands) return run_snapshots<64, bf16_t, float>(a, window, w0, nw, snap, st);
    return in_bf16 ? run_snapshots<64, bf16_t, _Float16>(a, window, w0, nw, snap, st)
                   : run_snapshots<64, float, float>(a, window, w0, nw, snap, st);
}

hipError_t chunk_dispatch(int d, bool in_bf16, bool out_bf16, bool qk_norm, int bv, const ChunkArgs& a, int nwin,
                          hipStream_t st, bool f32_operands) {
    if (d == 128) {
        if (in_bf16 && f32_operands) return run_norm<128, bf16_t, float>(a, out_bf16, qk_norm, nwin, bv, st);
        if (in_bf16) return run_norm<128, bf16_t, _Float16>(a, out_bf16, qk_norm, nwin, bv, st);
        return run_norm<128, float, float>(a, out_bf16, qk_norm, nwin, bv, st);
    }
    if (in_bf16 && f32_operands) return run_norm<64, bf16_t, float>(a, out_bf16, qk_norm, nwin, bv, st);
    if (in_bf16) return run_norm<64, bf16_t, _Float16>(a, out_bf16, qk_norm, nwin, bv, st);
    return run_norm<64, float, float>(a, out_bf16, qk_norm, nwin, bv, st);
}

// One partial max of |x| per block: grid-stride over the elements, then a
// shared-memory tree over the block's 256 threads.
template <typename T>
__global__ void __launch_bounds__(256) max_abs_kernel(const T* x, size_t n, float* block_max) {
    __shared__ float red[256];
    float m = 0.f;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        const float a = fabsf(to_f32(x[i]));
        m = a == a ? fmaxf(m, a) : __builtin_inff();
    }
    red[threadIdx.x] = m;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) block_max[blockIdx.x] = red[0];
}

hipError_t max_abs_dispatch(const void* x, size_t n, bool bf16, float* block_max, int nblocks, hipStream_t st) {
    if (bf16)
        hipLaunchKernelGGL((max_abs_kernel<bf16_t>), dim3(nblocks), dim3(256), 0, st, static_cast<const bf16_t*>(x),
                           n, block_max);
    else
        hipLaunchKernelGGL((max_abs_kernel<float>), dim3(nblocks), dim3(256), 0, st, static_cast<const float*>(x), n,
                           block_max);
    return hipGetLastError();
}

}  // namespace kda
