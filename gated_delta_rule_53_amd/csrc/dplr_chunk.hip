// dplr_chunk.hip -- chunked prefill of the general DPLR transition on gfx950.
//
// The transition KDA constrains ("Kimi Linear" page, "The constrained DPLR form
// and the chunkwise algorithm"): a diagonal gate plus a rank-one term whose two
// vectors a and b are independent of the key,
//     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,    o_t = S_t^T q_t.
// The rank-one term reads w_t = b_t^T S_{t-1}, the state before the token's own
// decay (KDA is the case a = beta k, b = alpha (.) k, write key beta k).
//
// Notation for one (sequence, head) and one chunk of n <= 64 tokens, rows r and
// columns i indexing tokens, c key channels; G_r = sum_{t<=r} log_alpha_t
// (chunk-local, per channel) and Gx_r = G_r - log_alpha_r:
//   Mba[r,i] = sum_c b_rc a_ic e^{Gx_rc - G_ic},  Mbk[r,i] likewise with k   (i < r)
//   Mqa[r,i] = sum_c q_rc a_ic e^{G_rc - G_ic},   Mqk[r,i] likewise with k   (i <= r)
//   T = (I + Mba)^-1,   Y = T (B e^{Gx}),   Z = (T Mbk) V
//   Qg = Q e^G,   Kh = K e^{G_last - G},   Ah = A e^{G_last - G},   gamma = e^{G_last}
// and between chunks, with the fp32 state S (dk x dv):
//   w = Z + Y S;   O = Qg S + Mqk V - Mqa w;   S <- Diag(gamma) S + Kh^T V - Ah^T w.
// Against KDA the gate no longer factors into one scaling of the key: four gated
// products instead of two (b sees the exclusive decay Gx, q the inclusive one),
// the extra product Mbk V, and a record that also carries Ah, V and the output
// products Mqk and Mqa.
//
// Gate products never divide by a cumulative decay.  Off-diagonal blocks split
// e^{G_r - G_i} at an anchor row m between i and r into a row factor
// e^{G_r - G_m} <= 1 and a column factor e^{G_m - G_i} <= 1: the 32 x 32 block
// below the diagonal (anchor 31), then the two 16 x 16 blocks below the
// diagonal of each half (anchors 15 and 47).  The 16 x 16 diagonal blocks use
// the last row of their first half as anchor, with factors up to the inverse of
// one eight-token decay; when that leaves the operands' range (fp16: 256, fp32:
// 2^64) the workgroup forms them instead with factors that are all <= 1: the
// later half against the earlier half at their boundary on matrix cores, the
// pairs inside each eight-row half as products of alpha over the pair's tokens.
// Matrix-core operands are fp16 for bf16 inputs and fp32 for fp32 inputs;
// accumulation, T and the state are fp32.
#include "kda_chunk_common.h"

#include <algorithm>

namespace kda {
namespace {

constexpr int DD = 128;  // key and value head dimension of this variant

// Per-chunk record (bytes).
template <typename OT>
struct DRec {
    static constexpr size_t TILE = (size_t)CH * DD * sizeof(OT);
    static constexpr size_t SQ = (size_t)CH * CH * sizeof(OT);
    static constexpr size_t Y = 0;                         // 64 x D, fragment order
    static constexpr size_t QG = align256(Y + TILE);       // 64 x D, fragment order
    static constexpr size_t KHT = align256(QG + TILE);     // D x 64, fragment order: Kh^T
    static constexpr size_t ANT = align256(KHT + TILE);    // D x 64, fragment order: -Ah^T
    static constexpr size_t MQK = align256(ANT + TILE);    // 64 x 64, fragment order
    static constexpr size_t NQA = align256(MQK + SQ);      // 64 x 64, fragment order: -Mqa
    static constexpr size_t Z = align256(NQA + SQ);        // [4 row tiles][D][16 rows]
    static constexpr size_t V = align256(Z + TILE);        // [4 row tiles][D][16 rows]
    static constexpr size_t GAM = align256(V + TILE);      // fp32 [D]
    static constexpr size_t BYTES = align256(GAM + DD * sizeof(float));
};

// LDS of the chunk-local kernel.  R_OP: the gate products of the half-blocks,
// then the operand rows of each set of gated products (128 rows: b, q, a, k
// scaled for one anchor), then T (fp32), then the channel-major right-hand sides
// B e^{Gx} and V.  R_A: Mba (fp32), later T as an fp16 operand.  R_M: Mbk stored
// transposed, -Mqa and Mqk (later T Mbk).
template <typename OT>
struct DCfg {
    static constexpr int NT = 512, NW = 8;
    static constexpr bool F16 = sizeof(OT) == 2;
    static constexpr int PD = Pad<OT>::v;
    static constexpr int DP = DD + PD;   // [row][channel] operand rows
    static constexpr int DP32 = DD + 4;  // fp32 operand rows of the all-factors-<=-1 diagonal form
    static constexpr int KP = CH + PD;   // [channel][token] rows
    static constexpr int MP = CH + PD;   // [64][64] OT matrices
    static constexpr int AP = CH + 1;    // [64][64] fp32 matrices
    static constexpr int THP = F16 ? MP : AP;
    static constexpr size_t SZ_F = (size_t)CH * AP * sizeof(float);
    static constexpr size_t SZ_RHS = (size_t)DD * KP * sizeof(OT);
    static constexpr size_t OFF_RHS = F16 ? 0 : SZ_F;  // fp32: T is read in place, before them
    static constexpr size_t SZ_OP = std::max(std::max((size_t)128 * DP * sizeof(OT), OFF_RHS + 2 * SZ_RHS),
                                             std::max(SZ_F, (size_t)64 * DP32 * sizeof(float)));
    static constexpr size_t R_A = align256(SZ_OP);
    static constexpr size_t R_M = R_A + SZ_F;
    static constexpr size_t SZ_M = (size_t)CH * MP * sizeof(OT);
    static constexpr size_t SMEM = R_M + 3 * SZ_M;
    static_assert(8 * DD * sizeof(float) <= 3 * SZ_M, "half-block products must fit R_M");
    static_assert(!F16 || (size_t)CH * THP * sizeof(OT) <= SZ_F, "the fp16 T operand must fit R_A");
};

constexpr float DPLR_F16_OPERAND_LIMIT = 6.0e4f;
constexpr float DPLR_F16_FACTOR_LIMIT = 256.f;
constexpr float DPLR_F32_FACTOR_LIMIT = 1.8446744e19f;  // 2^64

template <typename IT, typename OT>
__global__ void __launch_bounds__(512) dplr_local_kernel(ChunkArgs a) {
    using C = DCfg<OT>;
    using R = DRec<OT>;
    using FO = FragOrder<OT>;
    __shared__ __align__(16) unsigned char smem[C::SMEM];
    OT* sOp = reinterpret_cast<OT*>(smem);
    float* sOp32 = reinterpret_cast<float*>(smem);
    float* sT = reinterpret_cast<float*>(smem);
    OT* sBxT = reinterpret_cast<OT*>(smem + C::OFF_RHS);
    OT* sVT = reinterpret_cast<OT*>(smem + C::OFF_RHS + C::SZ_RHS);
    float* sA = reinterpret_cast<float*>(smem + C::R_A);
    OT* sTh = C::F16 ? reinterpret_cast<OT*>(smem + C::R_A) : reinterpret_cast<OT*>(smem);
    OT* sMbkT = reinterpret_cast<OT*>(smem + C::R_M);
    OT* sNqa = reinterpret_cast<OT*>(smem + C::R_M + C::SZ_M);
    OT* sMqk = reinterpret_cast<OT*>(smem + C::R_M + 2 * C::SZ_M);
    OT* sTM = sMqk;                                       // T Mbk, once Mqk is in the record
    float* sH = reinterpret_cast<float*>(smem + C::R_M);  // half-block gate products, first of all

    const int h = blockIdx.x, s = blockIdx.y / a.Wc, jl = blockIdx.y % a.Wc;
    int64_t tb, L;
    seq_bounds(a, s, tb, L);
    const int64_t c0 = (int64_t)(a.win * a.Wc + jl) * CH;
    if (c0 >= L) return;  // whole workgroup: no chunk here
    const int n = (int)min<int64_t>(CH, L - c0);
    const int64_t tok0 = tb + c0;
    const int H = a.H;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int gq = lane >> 4, li = lane & 15;
    // this thread: channels ch, ch + 1 of the eight rows of half-block hb
    const int hb = wave, r0 = 8 * hb, ch = 2 * lane;

    // ---- loads: gates first, then q, k, a, b, v (rows past the end read the
    // last valid row and are zeroed; their gates become 1) ----
    Pair8<IT> qq, kk, aa, bb, vv;
    float al[8][2];
    {
        const IT* q = static_cast<const IT*>(a.q);
        const IT* k = static_cast<const IT*>(a.k);
        const IT* v = static_cast<const IT*>(a.v);
        const IT* av = static_cast<const IT*>(a.dplr_a);
        const IT* bv = static_cast<const IT*>(a.dplr_b);
        size_t off[8];
        float g0[8], g1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            off[i] = ((size_t)(tok0 + min(r0 + i, n - 1)) * H + h) * DD + ch;
            g0[i] = __builtin_nontemporal_load(a.la + off[i]);
            g1[i] = __builtin_nontemporal_load(a.la + off[i] + 1);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) qq.load(i, q + off[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) kk.load(i, k + off[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) aa.load(i, av + off[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) bb.load(i, bv + off[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) vv.load(i, v + off[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            al[i][0] = fast_exp(g0[i]);
            al[i][1] = fast_exp(g1[i]);
        }
        if (n < CH) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (r0 + i >= n) {
                    al[i][0] = al[i][1] = 1.f;
                    qq.zero(i);
                    kk.zero(i);
                    aa.zero(i);
                    bb.zero(i);
                    vv.zero(i);
                }
        }
    }
    // products of alpha inside the half-block: p[i] over rows 0..i, px[i] over
    // rows 0..i-1, sf[i] over rows i+1..7 (all <= 1)
    float p[8][2], px[8][2], sf[8][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        px[0][e] = 1.f;
        p[0][e] = al[0][e];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            px[i][e] = p[i - 1][e];
            p[i][e] = p[i - 1][e] * al[i][e];
        }
        sf[7][e] = 1.f;
#pragma unroll
        for (int i = 6; i >= 0; --i) sf[i][e] = sf[i + 1][e] * al[i + 1][e];
    }
    *reinterpret_cast<float2*>(sH + hb * DD + ch) = make_float2(p[7][0], p[7][1]);
    lds_barrier();
    float Hq[8][2];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const float2 hv = *reinterpret_cast<const float2*>(sH + x * DD + ch);
        Hq[x][0] = hv.x;
        Hq[x][1] = hv.y;
    }
    // product of the half-block decays lo..hi (1 when empty)
    auto prodH = [&](int lo, int hi, int e) {
        float x = 1.f;
#pragma unroll
        for (int y = 0; y < 8; ++y)
            if (y >= lo && y <= hi) x *= Hq[y][e];
        return x;
    };
    // one 16 x 16 tile of a gated product into its matrix; type 0 Mba, 1 Mbk,
    // 2 Mqa (stored negated), 3 Mqk; mask 0 none, 1 strictly lower, 2 lower
    auto put_tile = [&](int type, int row0, int col0, const floatx4& acc, int mask) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int lr = 4 * gq + r;
            const bool keep = mask == 0 || (mask == 1 ? lr > li : lr >= li);
            const float x = keep ? acc[r] : 0.f;
            const int row = row0 + lr, col = col0 + li;
            if (type == 0)
                sA[row * C::AP + col] = x;
            else if (type == 1)
                sMbkT[col * C::MP + row] = from_f32<OT>(x);
            else if (type == 2)
                sNqa[row * C::MP + col] = from_f32<OT>(-x);
            else
                sMqk[row * C::MP + col] = from_f32<OT>(x);
        }
    };
    // operand rows of each set of products: b at 0.., q at 32.., a at 64.., k at 96..
    auto put_left = [&](int row, int i, float fb0, float fb1, float fq0, float fq1) {
        put2<OT>(sOp + row * C::DP + ch, bb.get(i, 0) * fb0, bb.get(i, 1) * fb1);
        put2<OT>(sOp + (32 + row) * C::DP + ch, qq.get(i, 0) * fq0, qq.get(i, 1) * fq1);
    };
    auto put_right = [&](int row, int i, float f0, float f1) {
        put2<OT>(sOp + (64 + row) * C::DP + ch, aa.get(i, 0) * f0, aa.get(i, 1) * f1);
        put2<OT>(sOp + (96 + row) * C::DP + ch, kk.get(i, 0) * f0, kk.get(i, 1) * f1);
    };
    auto round_tile = [&](int type, int lrow, int rrow) {
        floatx4 acc = zero4();
        mma_tile<OT>(acc, sOp + ((type < 2 ? 0 : 32) + lrow) * C::DP, C::DP,
                     sOp + ((type & 1 ? 96 : 64) + rrow) * C::DP, C::DP, DD, lane);
        return acc;
    };

    // ---- level 32: rows 32..63 against columns 0..31, anchor row 31 ----
    if (hb >= 4) {
        const float L0 = prodH(4, hb - 1, 0), L1 = prodH(4, hb - 1, 1);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            put_left(r0 + i - 32, i, L0 * px[i][0], L1 * px[i][1], L0 * p[i][0], L1 * p[i][1]);
    } else {
        const float R0 = prodH(hb + 1, 3, 0), R1 = prodH(hb + 1, 3, 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) put_right(r0 + i, i, R0 * sf[i][0], R1 * sf[i][1]);
    }
    lds_barrier();
    {
        // the blocks above the 16 x 16 diagonal are zero in Mbk, Mqa and Mqk (sH,
        // which shares their region, has been read by every thread)
        for (int idx = t; idx < 3 * 6 * 256; idx += C::NT) {
            const int m = idx / (6 * 256), b6 = (idx / 256) % 6, e = idx % 256;
            const int rb = b6 < 3 ? 0 : (b6 < 5 ? 1 : 2);
            const int cb = b6 < 3 ? b6 + 1 : (b6 < 5 ? b6 - 1 : 3);
            const int row = 16 * rb + (e >> 4), col = 16 * cb + (e & 15);
            if (m == 0)
                sMbkT[col * C::MP + row] = from_f32<OT>(0.f);
            else
                (m == 1 ? sNqa : sMqk)[row * C::MP + col] = from_f32<OT>(0.f);
        }
        for (int q2 = wave; q2 < 16; q2 += C::NW) {
            const int type = q2 >> 2, rt = (q2 >> 1) & 1, ct = q2 & 1;
            put_tile(type, 32 + 16 * rt, 16 * ct, round_tile(type, 16 * rt, 16 * ct), 0);
        }
    }
    lds_barrier();

    // ---- level 16: rows 16..31 against 0..15 (anchor 15), 48..63 against 32..47 (anchor 47) ----
    {
        const int half = hb >> 2, hq = hb & 3;
        if (hq >= 2) {
            const float L0 = prodH(4 * half + 2, hb - 1, 0), L1 = prodH(4 * half + 2, hb - 1, 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                put_left(16 * half + 8 * (hq - 2) + i, i, L0 * px[i][0], L1 * px[i][1], L0 * p[i][0], L1 * p[i][1]);
        } else {
            const float R0 = prodH(hb + 1, 4 * half + 1, 0), R1 = prodH(hb + 1, 4 * half + 1, 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) put_right(16 * half + 8 * hq + i, i, R0 * sf[i][0], R1 * sf[i][1]);
        }
    }
    lds_barrier();
    {
        const int type = wave >> 1, blk = wave & 1;
        put_tile(type, 16 + 32 * blk, 32 * blk, round_tile(type, 16 * blk, 16 * blk), 0);
    }

    // ---- diagonal 16 x 16 blocks, anchored at the last row of the first half ----
    // The first half's row factors and the second half's column factors are the
    // inverse of an eight-token decay at most: rcp = 1 / (the half-block's decay).
    float rcp[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) rcp[e] = __builtin_amdgcn_rcpf(p[7][e]);
    int wide;
    {
        const float fx = fmaxf(rcp[0], rcp[1]);
        float mx = 0.f;
        if (C::F16) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(qq.get(i, e)), fabsf(kk.get(i, e))),
                                         fmaxf(fabsf(aa.get(i, e)), fabsf(bb.get(i, e)))));
        }
        // also the barrier after the level-16 products
        wide = C::F16 ? __syncthreads_or(!(mx * fx <= DPLR_F16_OPERAND_LIMIT) || !(fx <= DPLR_F16_FACTOR_LIMIT))
                      : __syncthreads_or(!(fx <= DPLR_F32_FACTOR_LIMIT));
    }
    if (!wide) {
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            if ((hb >> 2) == pass) {
                const int hh = hb & 1, row0 = 16 * ((hb >> 1) & 1) + 8 * hh;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float m0 = hh ? 1.f : rcp[0], m1 = hh ? 1.f : rcp[1];
                    const float c0 = hh ? rcp[0] : 1.f, c1 = hh ? rcp[1] : 1.f;
                    put_left(row0 + i, i, px[i][0] * m0, px[i][1] * m1, p[i][0] * m0, p[i][1] * m1);
                    put_right(row0 + i, i, sf[i][0] * c0, sf[i][1] * c1);
                }
            }
            lds_barrier();
            {
                const int type = wave >> 1, blk = wave & 1, db = 2 * pass + blk;
                put_tile(type, 16 * db, 16 * db, round_tile(type, 16 * blk, 16 * blk), type < 2 ? 1 : 2);
            }
            lds_barrier();
        }
    } else {
        // Every factor <= 1.  Later half against earlier half: rows 8..15 carry
        // their decay since the boundary, rows 0..7 the decay after them up to it;
        // fp32 operands, one block at a time (b 0..15, q 16..31, a 32..47, k 48..63;
        // the other half's rows are zero, so the tile holds only those pairs).
#pragma unroll 1
        for (int db = 0; db < 4; ++db) {
            if ((hb >> 1) == db) {
                const int hh = hb & 1;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int row = 8 * hh + i;
                    const float l0 = hh ? 1.f : 0.f, r1 = hh ? 0.f : 1.f;
                    put2<float>(sOp32 + row * C::DP32 + ch, bb.get(i, 0) * px[i][0] * l0,
                                bb.get(i, 1) * px[i][1] * l0);
                    put2<float>(sOp32 + (16 + row) * C::DP32 + ch, qq.get(i, 0) * p[i][0] * l0,
                                qq.get(i, 1) * p[i][1] * l0);
                    put2<float>(sOp32 + (32 + row) * C::DP32 + ch, aa.get(i, 0) * sf[i][0] * r1,
                                aa.get(i, 1) * sf[i][1] * r1);
                    put2<float>(sOp32 + (48 + row) * C::DP32 + ch, kk.get(i, 0) * sf[i][0] * r1,
                                kk.get(i, 1) * sf[i][1] * r1);
                }
            }
            lds_barrier();
            if (wave < 4) {
                const int type = wave;
                floatx4 acc = zero4();
                const float* pa = sOp32 + ((type < 2 ? 0 : 16) + li) * C::DP32 + gq;
                const float* pb = sOp32 + ((type & 1 ? 48 : 32) + li) * C::DP32 + gq;
#pragma unroll 4
                for (int k0 = 0; k0 < DD; k0 += 4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0], pb[k0], acc, 0, 0, 0);
                put_tile(type, 16 * db, 16 * db, acc, 0);
            }
            lds_barrier();
        }
        // Pairs inside this wave's eight rows: the decay over the pair's tokens as a
        // running product, summed over the wave's 128 channels.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float f[2] = {1.f, 1.f};  // prod of alpha over rows i+1 .. r-1
#pragma unroll
            for (int r = i; r < 8; ++r) {
                float xba = 0.f, xbk = 0.f, xqa = 0.f, xqk = 0.f;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float fq = r == i ? 1.f : f[e] * al[r][e];
                    if (r > i) {
                        const float bl = bb.get(r, e) * f[e];
                        xba += bl * aa.get(i, e);
                        xbk += bl * kk.get(i, e);
                    }
                    const float ql = qq.get(r, e) * fq;
                    xqa += ql * aa.get(i, e);
                    xqk += ql * kk.get(i, e);
                    if (r > i) f[e] = fq;
                }
                xqa = row_sum<64>(xqa);
                xqk = row_sum<64>(xqk);
                if (r > i) {
                    xba = row_sum<64>(xba);
                    xbk = row_sum<64>(xbk);
                }
                if (lane == 0) {
                    const int row = r0 + r, col = r0 + i;
                    if (r > i) {
                        sA[row * C::AP + col] = xba;
                        sMbkT[col * C::MP + row] = from_f32<OT>(xbk);
                    }
                    sNqa[row * C::MP + col] = from_f32<OT>(-xqa);
                    sMqk[row * C::MP + col] = from_f32<OT>(xqk);
                }
            }
        }
        lds_barrier();
    }

    // ---- Mqk and -Mqa to the record, then T = (I + Mba)^-1 ----
    unsigned char* rec = a.rec + ((size_t)(s * a.Wc + jl) * H + h) * a.rec_bytes;
    {
        OT* rM = reinterpret_cast<OT*>(rec + R::MQK);
        OT* rN = reinterpret_cast<OT*>(rec + R::NQA);
        for (int f = t; f < 2 * CH * CH / FO::KE; f += C::NT) {  // one lane slot of one fragment per step
            const int g = f % (CH * CH / FO::KE), which = f / (CH * CH / FO::KE);
            const int l = g & 63, k2 = (g >> 6) % (CH / FO::KS), rt = (g >> 6) / (CH / FO::KS);
            const OT* src = (which ? sNqa : sMqk) + (16 * rt + (l & 15)) * C::MP + k2 * FO::KS + (l >> 4) * FO::KE;
            OT* dst = (which ? rN : rM) + (size_t)g * FO::KE;
            if constexpr (FO::KE == 8)
                *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
            else
                dst[0] = src[0];
        }
    }
    ut_inverse64<C::AP, C::NW>(sT, sA, wave, lane);
    if (C::F16) {
        for (int idx = t; idx < CH * CH / 8; idx += C::NT) {
            const int r = idx / 8, i = (idx % 8) * 8;
            float x[8];
            const bool upper = (i >> 4) > (r >> 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = upper ? 0.f : sT[r * C::AP + i + e];
            store8<OT>(sTh + r * C::THP + i, x);
        }
    } else {
        for (int idx = t; idx < CH * CH; idx += C::NT) {
            const int r = idx / CH, i = idx % CH;
            if ((i >> 4) > (r >> 4)) sT[r * C::AP + i] = 0.f;
        }
    }
    __syncthreads();

    // ---- channel-major B e^{Gx} and V; the record's register-held parts ----
    {
        float Eb[2], Sa[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            Eb[e] = prodH(0, hb - 1, e);  // e^{G} of the row before this half-block
            Sa[e] = prodH(hb + 1, 7, e);  // decay of the half-blocks after it
        }
        float x0[8], x1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x0[i] = bb.get(i, 0) * (Eb[0] * px[i][0]);
            x1[i] = bb.get(i, 1) * (Eb[1] * px[i][1]);
        }
        store8<OT>(sBxT + (size_t)ch * C::KP + r0, x0);
        store8<OT>(sBxT + (size_t)(ch + 1) * C::KP + r0, x1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x0[i] = vv.get(i, 0);
            x1[i] = vv.get(i, 1);
        }
        store8<OT>(sVT + (size_t)ch * C::KP + r0, x0);
        store8<OT>(sVT + (size_t)(ch + 1) * C::KP + r0, x1);
        OT* rV = reinterpret_cast<OT*>(rec + R::V);
        store8<OT>(rV + ((size_t)(hb >> 1) * DD + ch) * 16 + 8 * (hb & 1), x0);
        store8<OT>(rV + ((size_t)(hb >> 1) * DD + ch + 1) * 16 + 8 * (hb & 1), x1);
        // Qg: the two channels of a row are adjacent in fragment order (ch is even)
        OT* rQ = reinterpret_cast<OT*>(rec + R::QG);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float f0 = Eb[0] * p[i][0], f1 = Eb[1] * p[i][1];
            if (C::F16) {
                put2<OT>(rQ + FO::idx(r0 + i, ch, DD), qq.get(i, 0) * f0, qq.get(i, 1) * f1);
            } else {
                rQ[FO::idx(r0 + i, ch, DD)] = from_f32<OT>(qq.get(i, 0) * f0);
                rQ[FO::idx(r0 + i, ch + 1, DD)] = from_f32<OT>(qq.get(i, 1) * f1);
            }
        }
        // Kh^T and -Ah^T: 8 consecutive tokens of a channel are contiguous in fragment order (fp16)
        OT* rK = reinterpret_cast<OT*>(rec + R::KHT);
        OT* rA = reinterpret_cast<OT*>(rec + R::ANT);
        float y0[8], y1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float f0 = sf[i][0] * Sa[0], f1 = sf[i][1] * Sa[1];
            x0[i] = kk.get(i, 0) * f0;
            x1[i] = kk.get(i, 1) * f1;
            y0[i] = -aa.get(i, 0) * f0;
            y1[i] = -aa.get(i, 1) * f1;
        }
        if (C::F16) {
            store8<OT>(rK + FO::idx(ch, r0, CH), x0);
            store8<OT>(rK + FO::idx(ch + 1, r0, CH), x1);
            store8<OT>(rA + FO::idx(ch, r0, CH), y0);
            store8<OT>(rA + FO::idx(ch + 1, r0, CH), y1);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                rK[FO::idx(ch, r0 + i, CH)] = from_f32<OT>(x0[i]);
                rK[FO::idx(ch + 1, r0 + i, CH)] = from_f32<OT>(x1[i]);
                rA[FO::idx(ch, r0 + i, CH)] = from_f32<OT>(y0[i]);
                rA[FO::idx(ch + 1, r0 + i, CH)] = from_f32<OT>(y1[i]);
            }
        }
        if (hb == 0) {
            float* rG = reinterpret_cast<float*>(rec + R::GAM);
            *reinterpret_cast<float2*>(rG + ch) = make_float2(prodH(0, 7, 0), prodH(0, 7, 1));
        }
    }
    __syncthreads();

    // ---- Y = T (B e^{Gx}) to the record, and T Mbk ----
    constexpr int KS = Mma<OT>::KSTEP;
    {
        OT* rY = reinterpret_cast<OT*>(rec + R::Y);
        for (int q2 = wave; q2 < 42; q2 += C::NW) {
            floatx4 acc = zero4();
            if (q2 < 32) {
                const int rb = q2 >> 3, ct = q2 & 7;
                const int K = ((16 * (rb + 1) + KS - 1) / KS) * KS;
                // Y^T tile: lane holds channels 16ct+4gq..+3 of row 16rb+li, 4 consecutive
                // elements in fragment order
                mma_tile<OT>(acc, sBxT + (16 * ct) * C::KP, C::KP, sTh + (16 * rb) * C::THP, C::THP, K, lane);
                if (C::F16) {
                    store4<OT>(rY + FO::idx(16 * rb + li, 16 * ct + 4 * gq, DD), acc);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rY[FO::idx(16 * rb + li, 16 * ct + 4 * gq + e, DD)] = from_f32<OT>(acc[e]);
                }
            } else {
                const int x = q2 - 32;  // lower tiles (rb, cb), cb <= rb
                const int rb = x < 1 ? 0 : (x < 3 ? 1 : (x < 6 ? 2 : 3));
                const int cb = x - rb * (rb + 1) / 2;
                const int K = ((16 * (rb + 1) + KS - 1) / KS) * KS;
                mma_tile<OT>(acc, sTh + (16 * rb) * C::THP, C::THP, sMbkT + (16 * cb) * C::MP, C::MP, K, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) sTM[(16 * rb + 4 * gq + r) * C::MP + 16 * cb + li] = from_f32<OT>(acc[r]);
            }
        }
    }
    __syncthreads();

    // ---- Z = (T Mbk) V to the record ----
    {
        OT* rZ = reinterpret_cast<OT*>(rec + R::Z);
        for (int q2 = wave; q2 < 32; q2 += C::NW) {
            const int rb = q2 >> 3, ct = q2 & 7;
            const int K = ((16 * (rb + 1) + KS - 1) / KS) * KS;
            floatx4 acc = zero4();
            mma_tile<OT>(acc, sTM + (16 * rb) * C::MP, C::MP, sVT + (16 * ct) * C::KP, C::KP, K, lane);
            store4<OT>(rZ + ((size_t)rb * DD + 16 * ct + li) * 16 + 4 * gq, acc);
        }
    }
}

// ---------------------------------------------------------------------------
// State pass: one workgroup of 8 waves per (sequence, head, slice of BV value
// columns).  Waves 0..3 carry the state: for chunk j they form w_j = Z_j + Y_j S_j
// and S_{j+1} = Diag(gamma_j) S_j + Kh_j^T V_j - Ah_j^T w_j.  Waves 4..7 form
// O_j = Qg_j S_j + Mqk_j V_j - Mqa_j w_j.  S_j, V_j and w_j pass through
// double-buffered LDS tiles; two barriers per chunk.
// ---------------------------------------------------------------------------
template <int BV, typename OT, typename OUT>
__global__ void __launch_bounds__(512) dplr_inter_kernel(ChunkArgs a) {
    using R = DRec<OT>;
    using FR = Frag<OT>;
    using FT = typename FR::T;
    using FO = FragOrder<OT>;
    constexpr int KS = Mma<OT>::KSTEP;
    constexpr int NFD = DD / KS;  // fragments along a D-long row
    constexpr int NFT = CH / KS;  // fragments along a 64-long row
    constexpr int RT = DD / 64;   // 16-row state tiles per chain wave
    constexpr int CT = BV / 16;
    constexpr int PD = Pad<OT>::v;
    constexpr int SP = DD + PD;
    constexpr int UP = CH + PD;
    __shared__ __align__(16) OT sS[2][BV * SP];
    __shared__ __align__(16) OT sW[2][BV * UP];
    __shared__ __align__(16) OT sV[2][BV * UP];

    const int H = a.H;
    const int NH = a.N * H;
    const int u = blockIdx.x % NH, z = blockIdx.x / NH;
    const int s = u / H, h = u % H;
    int64_t tb, L;
    seq_bounds(a, s, tb, L);
    const int nchunks = (int)((L + CH - 1) / CH);
    const int jb = a.win * a.Wc;
    const int je = min(nchunks, jb + a.Wc);
    if (jb >= je && a.win > 0) return;  // the state left by the last window stands

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const bool chain = wave < 4;
    const int w = wave & 3;
    const int gq = lane >> 4, li = lane & 15;
    const int col0 = z * BV;
    OUT* out = static_cast<OUT*>(a.out);
    auto rec_of = [&](int j) { return a.rec + ((size_t)(s * a.Wc + (j - jb)) * H + h) * a.rec_bytes; };

    if (chain) {
        floatx4 Sacc[RT][CT];
        const float* src = a.win == 0 ? a.init : a.state_buf;
        if (src) src += (size_t)u * DD * DD;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = w * (DD / 4) + 16 * rt + 4 * gq + r;
                    Sacc[rt][ct][r] = src ? src[(size_t)row * DD + col0 + 16 * ct + li] : 0.f;
                }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                store4<OT>(&sS[0][(16 * ct + li) * SP + w * (DD / 4) + 16 * rt + 4 * gq], Sacc[rt][ct]);

        struct ChainBuf {
            floatx4 V[CT];
            floatx4 Z[CT];
            FT Y[NFD];
            FT K[RT][NFT];
            FT A[RT][NFT];
            float G;  // gamma of state row w*D/4 + lane % (D/4)
        };
        auto load = [&](ChainBuf& f, int j) {
            const unsigned char* rec = rec_of(j);
            const OT* rV = reinterpret_cast<const OT*>(rec + R::V);
            const OT* rZ = reinterpret_cast<const OT*>(rec + R::Z);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) f.V[ct] = load4<OT>(rV + ((size_t)w * DD + col0 + 16 * ct + li) * 16 + 4 * gq);
            f.G = reinterpret_cast<const float*>(rec + R::GAM)[w * (DD / 4) + lane % (DD / 4)];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) f.Z[ct] = load4<OT>(rZ + ((size_t)w * DD + col0 + 16 * ct + li) * 16 + 4 * gq);
            const OT* rY = reinterpret_cast<const OT*>(rec + R::Y);
#pragma unroll
            for (int e = 0; e < NFD; ++e) f.Y[e] = FR::load(rY + FO::frag(w, e, lane, DD), 0);
            const OT* rK = reinterpret_cast<const OT*>(rec + R::KHT);
            const OT* rA = reinterpret_cast<const OT*>(rec + R::ANT);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int e = 0; e < NFT; ++e) {
                    f.K[rt][e] = FR::load(rK + FO::frag(w * RT + rt, e, lane, CH), 0);
                    f.A[rt][e] = FR::load(rA + FO::frag(w * RT + rt, e, lane, CH), 0);
                }
        };
        auto stage_v = [&](const ChainBuf& f, int buf) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) store4<OT>(sV[buf] + (16 * ct + li) * UP + 16 * w + 4 * gq, f.V[ct]);
        };
        auto step = [&](ChainBuf& f, const ChainBuf& fn, int j) {
            const int cur = (j - jb) & 1;
            float g[RT][4];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) g[rt][r] = __shfl(f.G, 16 * rt + 4 * gq + r);
            lds_barrier();  // S_j in sS[cur], V_j in sV[cur]
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                floatx4 acc = f.Z[ct];
                const OT* bt = sS[cur] + (16 * ct + li) * SP;
#pragma unroll
                for (int e = 0; e < NFD; ++e) acc = FR::mma(f.Y[e], bt + e * KS, gq, acc);
                store4<OT>(sW[cur] + (16 * ct + li) * UP + 16 * w + 4 * gq, acc);
            }
            lds_barrier();  // w_j in sW[cur]
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sacc[rt][ct][r] *= g[rt][r];
                    const OT* bv = sV[cur] + (16 * ct + li) * UP;
                    const OT* bw = sW[cur] + (16 * ct + li) * UP;
#pragma unroll
                    for (int e = 0; e < NFT; ++e) Sacc[rt][ct] = FR::mma(f.K[rt][e], bv + e * KS, gq, Sacc[rt][ct]);
#pragma unroll
                    for (int e = 0; e < NFT; ++e) Sacc[rt][ct] = FR::mma(f.A[rt][e], bw + e * KS, gq, Sacc[rt][ct]);
                }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    store4<OT>(sS[cur ^ 1] + (16 * ct + li) * SP + w * (DD / 4) + 16 * rt + 4 * gq, Sacc[rt][ct]);
            stage_v(fn, cur ^ 1);  // V_{j+1}
        };
        if (jb < je) {
            ChainBuf buf[2];
            load(buf[0], jb);
            stage_v(buf[0], 0);
            for (int j0 = jb; j0 < je; j0 += 2) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int j = j0 + p;
                    load(buf[p ^ 1], min(j + 1, je - 1));
                    if (j < je) step(buf[p], buf[p ^ 1], j);
                }
            }
        }
        float* dst = a.state_buf + (size_t)u * DD * DD;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = w * (DD / 4) + 16 * rt + 4 * gq + r;
                    dst[(size_t)row * DD + col0 + 16 * ct + li] = Sacc[rt][ct][r];
                }
    } else {
        struct OutBuf {
            FT Q[NFD];
            FT M[NFT];
            FT N[NFT];
        };
        auto load = [&](OutBuf& f, int j) {
            const unsigned char* rec = rec_of(j);
            const OT* rQ = reinterpret_cast<const OT*>(rec + R::QG);
            const OT* rM = reinterpret_cast<const OT*>(rec + R::MQK);
            const OT* rN = reinterpret_cast<const OT*>(rec + R::NQA);
#pragma unroll
            for (int e = 0; e < NFD; ++e) f.Q[e] = FR::load(rQ + FO::frag(w, e, lane, DD), 0);
#pragma unroll
            for (int e = 0; e < NFT; ++e) {
                f.M[e] = FR::load(rM + FO::frag(w, e, lane, CH), 0);
                f.N[e] = FR::load(rN + FO::frag(w, e, lane, CH), 0);
            }
        };
        auto step = [&](const OutBuf& f, int j) {
            const int cur = (j - jb) & 1;
            floatx4 acc[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                acc[ct] = zero4();
                const OT* bs = sS[cur] + (16 * ct + li) * SP;
                const OT* bv = sV[cur] + (16 * ct + li) * UP;
#pragma unroll
                for (int e = 0; e < NFD; ++e) acc[ct] = FR::mma(f.Q[e], bs + e * KS, gq, acc[ct]);
#pragma unroll
                for (int e = 0; e < NFT; ++e) acc[ct] = FR::mma(f.M[e], bv + e * KS, gq, acc[ct]);
            }
            lds_barrier();  // w_j in sW[cur]
            const int n = (int)min<int64_t>(CH, L - (int64_t)j * CH);
            const int64_t tok0 = tb + (int64_t)j * CH;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const OT* bw = sW[cur] + (16 * ct + li) * UP;
#pragma unroll
                for (int e = 0; e < NFT; ++e) acc[ct] = FR::mma(f.N[e], bw + e * KS, gq, acc[ct]);
                OUT* o = out + ((size_t)(tok0 + 16 * w + 4 * gq) * H + h) * DD + col0 + 16 * ct + li;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * w + 4 * gq + r < n) store_out(o + (size_t)r * H * DD, acc[ct][r]);
            }
        };
        if (jb < je) {
            OutBuf buf[2];
            load(buf[0], jb);
            for (int j0 = jb; j0 < je; j0 += 2) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int j = j0 + p;
                    if (j < je) lds_barrier();  // S_j in sS[cur], V_j in sV[cur]
                    load(buf[p ^ 1], min(j + 1, je - 1));
                    if (j < je) step(buf[p], j);
                }
            }
        }
    }
}

template <typename IT, typename OT, typename OUT, int BV>
hipError_t run_dplr(const ChunkArgs& base, int nwin, hipStream_t st) {
    const int units = base.N * base.H;
    for (int w = 0; w < nwin; ++w) {
        ChunkArgs a = base;
        a.win = w;
        hipLaunchKernelGGL((dplr_local_kernel<IT, OT>), dim3(a.H, a.N * a.Wc), dim3(512), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((dplr_inter_kernel<BV, OT, OUT>), dim3(units * (DD / BV)), dim3(512), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename IT, typename OT, typename OUT>
hipError_t run_dplr_bv(const ChunkArgs& a, int nwin, int bv, hipStream_t st) {
    if (bv == 16) return run_dplr<IT, OT, OUT, 16>(a, nwin, st);
    return run_dplr<IT, OT, OUT, 32>(a, nwin, st);
}

}  // namespace

size_t dplr_record_bytes(bool in_bf16) { return in_bf16 ? DRec<_Float16>::BYTES : DRec<float>::BYTES; }

int dplr_value_slice(bool in_bf16, int64_t units) {
    return in_bf16 && chunk_value_slice(DD, units) != 16 ? 32 : 16;
}

hipError_t dplr_dispatch(bool in_bf16, bool out_bf16, int bv, const ChunkArgs& a, int nwin, hipStream_t st) {
    if (in_bf16) {
        if (out_bf16) return run_dplr_bv<bf16_t, _Float16, bf16_t>(a, nwin, bv, st);
        return run_dplr_bv<bf16_t, _Float16, float>(a, nwin, bv, st);
    }
    // fp32 operands: the 16-column slice only (the wider one would spill registers)
    if (out_bf16) return run_dplr<float, float, bf16_t, 16>(a, nwin, st);
    return run_dplr<float, float, float, 16>(a, nwin, st);
}

}  // namespace kda
