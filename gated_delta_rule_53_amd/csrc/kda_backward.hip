// kda_backward.hip -- reverse mode of the chunked KDA prefill (gfx950, wave64).
//
// The gradients of L = sum(dO * O) + sum(dS_T * S_T) with respect to q, k, v,
// log_alpha, beta and the initial state, through the chunkwise form of the
// recurrence ("Kimi Linear" page, "The constrained DPLR form and the chunkwise
// algorithm").  Per chunk j with state S_j (entering the chunk), G the
// inclusive cumulative log-gate inside the chunk, Kg = K e^G, Qg = Q e^G,
// Kh = K e^{G_last - G}, gamma = e^{G_last}, A0 the strictly lower 64x64
// product A0[r][i] = sum_c k_rc k_ic e^{G_rc - G_ic}, Atil = diag(beta) A0,
// P the inclusive lower product with q in place of the row's k,
// T = (I + Atil)^-1, Bk = diag(beta) Kg, Bv = diag(beta) V, W = T Bk,
// Ut = T Bv:
//     U = Ut - W S_j,  O = Qg S_j + P U,  S_{j+1} = Diag(gamma) S_j + Kh^T U.
// Walking the chunks backwards with dS = dL/dS_{j+1}:
//     dU  = P^T dO + Kh dS
//     dS_j = Qg^T dO + Diag(gamma) dS - W^T dU
// and inside the chunk
//     dQg = dO S_j^T,  dP = tril(dO U^T),  dKh = U dS^T,  dgamma = rowsum(S_j o dS),
//     dW = -dU S_j^T,  dT = dW Bk^T + dU Bv^T,  dBk = T^T dW,  dBv = T^T dU,
//     dAtil = -T^T dT T^T (strictly lower),
// and the decay-weighted products of dP and diag(beta) dAtil with K and Q
// (row and column forms, below) carry the rest to q, k and G; dlog_alpha is
// the reverse cumulative sum of dG over the chunk's rows.
//
// Kernels (all fp32 arithmetic, fp32 matrix cores):
//   chunk_local_kernel + chunk_inter_kernel (the forward's, with state
//     snapshots): S_j and U_j for every chunk, U_j as the state pass forms it
//     (the U that carried S_j to S_{j+1});
//   bwd_prep_kernel   one 512-thread workgroup per (chunk, head): G, A0, P, T,
//                     W, Qg, Kh, gamma -> an fp32 record (T, A0, G row-major for
//                     the local pass; P^T, Kh, Qg^T, -W^T and gamma in the
//                     chain's matrix-core order);
//   bwd_chain_kernel  one 256-thread workgroup per (sequence, head, 16 value
//                     columns): the reverse chain over chunks, writing dS_{j+1}
//                     and dU_j, each chunk's operands loaded during the previous;
//   bwd_local_kernel  one 512-thread workgroup per (chunk, head): every
//                     parameter gradient.
//
// Decay factors e^{G_r - G_i} of the pairwise products are split about an
// anchor row so each matrix-core operand carries one bounded factor: for a
// 16-row block pair the first row of the later block (both factors <= 1), for a
// diagonal block its ninth row (factors bounded by eight tokens of decay).
#include "kda_chunk_common.h"

#include <type_traits>

namespace kda {

namespace {

// A diagonal 16-row block's single anchor (its ninth row) needs exponents up to the
// gate's decay over eight rows in both directions; past kWideExp (fp32 operands keep
// their products exact to far beyond what matters) the block is formed level by
// level instead: a pair (r, i) is formed where r and i first fall into different
// halves of an aligned sub-block of 16, 8, 4 or 2 rows, anchored at that
// sub-block's middle row, so every exponent is at most 0 and any gate is in range.
constexpr float kWideExp = 60.f;

constexpr int BW_T = 512;  // threads of the prep kernel (8 waves)
constexpr int BW_W = BW_T / 64;
constexpr int BL_T = 512;  // threads of the local kernel (8 waves)
constexpr int BL_W = BL_T / 64;

// Operands of one wave of the reverse chain for one chunk, in the order its
// matrix-core steps consume them.  Reduction index k of a part (k = 16 b + 4 g + e)
// is fed by lane l = li + 16 g at step 4 b + e of that part, so the four steps of
// block b take one float4 per lane (k = 16 b + 4 g .. +3) and the B operand, kept
// transposed in LDS, is one 16-byte read per lane as well.  Wave w owns dU rows
// 16w .. 16w+15 (parts P^T over the chunk's rows, then Kh over the key channels)
// and NRT 16-row tiles of dS at rows w D/4 + 16 rt (parts Qg^T, then -W^T, over
// the chunk's rows); after the steps, one float4 per tile holds gamma of the
// lane's four dS rows.
template <int D>
struct ChainRec {
    static constexpr int NRT = D / 64;
    static constexpr int EP = CH / 4, EK = D / 4, EQ = CH / 4;
    static constexpr int E = EP + EK + NRT * 2 * EQ;
    static constexpr int Q4 = E / 4 + NRT;
    static constexpr int FLOATS = 4 * Q4 * 64 * 4;
    __device__ static int at(int w, int e, int lane) { return ((w * Q4 + (e >> 2)) * 64 + lane) * 4 + (e & 3); }
    // step offset and lane group of reduction index k within a part
    __device__ static int ks(int k) { return 4 * (k >> 4) + (k & 3); }
    __device__ static int kg(int k) { return (k >> 2) & 3; }
    // dS tile of key channel c: wave, tile, and the step base of its Qg^T part
    __device__ static int wave_of(int c) { return c / (D / 4); }
    __device__ static int tile_of(int c) { return (c % (D / 4)) >> 4; }
    __device__ static int qbase(int c) { return EP + EK + tile_of(c) * 2 * EQ; }
};

// fp32 record of one (chunk, head), offsets in floats: what the local pass
// reads row-major, then the chain's operands
// The same operands as fp16 matrix-core fragments (bf16 inputs): per wave, the
// 16 x 32 A fragments of P^T (two, over the chunk's rows), Kh (D / 32, over the
// key channels), and for each dS tile those of Qg^T and -W^T (two each, over
// the chunk's rows); lane l = li + 16 g of fragment f holds reduction indices
// 32 (f - base) + 8 g .. + 7 of A-row li, 16 bytes.  gamma follows as fp32, one
// float4 per tile and lane (the lane's four dS rows).
template <int D>
struct ChainRec16 {
    static constexpr int NRT = D / 64;
    static constexpr int FK = D / 32;
    static constexpr int F = 2 + FK + 4 * NRT;           // fragments per wave
    static constexpr int GAM = 4 * F * 64 * 8 / 2;        // float offset of gamma
    static constexpr int FLOATS = GAM + 4 * NRT * 64 * 4;
    static constexpr int FKH = 2;                          // first Kh fragment
    __device__ static int fq(int rt) { return 2 + FK + 4 * rt; }      // first Qg^T fragment of tile rt
    __device__ static int fw(int rt) { return 2 + FK + 4 * rt + 2; }  // first -W^T fragment of tile rt
    // half offset of reduction index k of A-row li, in the fragments of wave w from fb
    __device__ static int at(int w, int fb, int k, int li) {
        return ((w * F + fb + (k >> 5)) * 64 + li + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
    }
    __device__ static int gam(int w, int rt, int lane, int r) { return GAM + ((w * NRT + rt) * 64 + lane) * 4 + r; }
};

template <int D>
struct BRec {
    static constexpr size_t T = 0;
    static constexpr size_t A0 = T + CH * CH;
    static constexpr size_t U = A0 + CH * CH;  // U = Ut - W S_j, stored by the recompute's state pass
    static constexpr size_t G = U + CH * D;
    static constexpr size_t CR = G + CH * D;
    static constexpr size_t FLOATS = CR + ChainRec<D>::FLOATS;
    static_assert(ChainRec16<D>::FLOATS <= ChainRec<D>::FLOATS, "fp16 chain operands fit the chain region");
    static_assert(U % 4 == 0 && FLOATS % 4 == 0, "the state pass stores U as 16-byte aligned float4s");
};

__device__ __forceinline__ void seq_range(const ChunkArgs& a, int s, int64_t& t0, int64_t& L) {
    if (a.cu) {
        t0 = a.cu[s];
        L = (int64_t)a.cu[s + 1] - t0;
    } else {
        t0 = (int64_t)s * a.T;
        L = a.T;
    }
}

template <typename X>
__device__ __forceinline__ float ld(const X* p, size_t i) {
    return to_f32(p[i]);
}

// four consecutive elements from p + i (i % 4 == 0), as fp32
__device__ __forceinline__ float4 ld4(const float* p, size_t i) { return *reinterpret_cast<const float4*>(p + i); }
__device__ __forceinline__ float4 ld4(const bf16_t* p, size_t i) {
    const uint2 w = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
}

// One 16x16 fp32 tile product acc += sum_k A(m, k) B(k, n), k = 0 .. K-1,
// with lane l feeding A(m0 + (l & 15), k) and B(k, n0 + (l & 15)) through the loaders;
// acc[r] of lane l ends as C(m0 + 4 (l >> 4) + r, n0 + (l & 15)).  K advances in
// groups of 4 GS (K % (4 GS) == 0) whose 2 GS operand loads are issued before their
// GS products, so the latency of loads from memory overlaps instead of adding up.
template <int GS = 4, typename FA, typename FB>
__device__ __forceinline__ void tile_f32(floatx4& acc, int K, int lane, FA&& a, FB&& b) {
    const int g = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 4 * GS) {
        float x[GS], y[GS];
#pragma unroll
        for (int e = 0; e < GS; ++e) {
            x[e] = a(k0 + 4 * e + g);
            y[e] = b(k0 + 4 * e + g);
        }
#pragma unroll
        for (int e = 0; e < GS; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e], y[e], acc, 0, 0, 0);
    }
}

// The same product with operands fetched four reduction indices at a time: the
// loaders return A(m0 + (l & 15), k .. k+3) and B(k .. k+3, n0 + (l & 15)) for
// k = k0 + 4 (l >> 4), and the four components feed four consecutive matrix-core
// steps (lane group g supplies index k0 + 4 g + e at step e; A and B agree, so
// the sum is the same).  K % (16 GS) == 0.
template <int GS = 2, typename FA, typename FB>
__device__ __forceinline__ void tile_f32_v(floatx4& acc, int K, int lane, FA&& a, FB&& b) {
    const int g4 = 4 * (lane >> 4);
    for (int k0 = 0; k0 < K; k0 += 16 * GS) {
        float4 x[GS], y[GS];
#pragma unroll
        for (int e = 0; e < GS; ++e) {
            x[e] = a(k0 + 16 * e + g4);
            y[e] = b(k0 + 16 * e + g4);
        }
#pragma unroll
        for (int e = 0; e < GS; ++e) {
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e].x, y[e].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e].y, y[e].y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e].z, y[e].z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e].w, y[e].w, acc, 0, 0, 0);
        }
    }
}

// Two products of one 16x16 tile shape, x += A1 B1 and y += A2 B2 (operands as for
// tile_f32_v), in one loop that also adds to d this lane's share of
// sum_k B1(k, n) B2(k, n) (its four reduction indices per 16).
template <int GS, typename FA1, typename FB1, typename FA2, typename FB2>
__device__ __forceinline__ void tile2_f32_v(floatx4& x, floatx4& y, float& d, int K, int lane, FA1&& a1, FB1&& b1,
                                            FA2&& a2, FB2&& b2) {
    const int g4 = 4 * (lane >> 4);
    for (int k0 = 0; k0 < K; k0 += 16 * GS) {
        float4 p[GS], q[GS], u[GS], w[GS];
#pragma unroll
        for (int e = 0; e < GS; ++e) {
            p[e] = a1(k0 + 16 * e + g4);
            q[e] = b1(k0 + 16 * e + g4);
            u[e] = a2(k0 + 16 * e + g4);
            w[e] = b2(k0 + 16 * e + g4);
        }
#pragma unroll
        for (int e = 0; e < GS; ++e) {
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(p[e].x, q[e].x, x, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(u[e].x, w[e].x, y, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(p[e].y, q[e].y, x, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(u[e].y, w[e].y, y, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(p[e].z, q[e].z, x, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(u[e].z, w[e].z, y, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(p[e].w, q[e].w, x, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(u[e].w, w[e].w, y, 0, 0, 0);
            d += q[e].x * w[e].x + q[e].y * w[e].y + q[e].z * w[e].z + q[e].w * w[e].w;
        }
    }
}

__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a row (lanes 16 g .. 16 g + 15), in every lane of the
// row: lane pairs, quads, then the mirrored half-row and row.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}

}  // namespace

// ---------------------------------------------------------------------------
// prep: the chunk's forward quantities in fp32
// ---------------------------------------------------------------------------
template <int D, typename IT>
__global__ void __launch_bounds__(BW_T) bwd_prep_kernel(ChunkArgs a, float* brec) {
    using R = BRec<D>;
    using C = ChainRec<D>;
    using C16 = ChainRec16<D>;
    constexpr bool H16 = std::is_same<IT, bf16_t>::value;  // chain operands as fp16 fragments
    constexpr int DP = D + 1;
    constexpr int AP = CH + 1;
    // q and k are staged in their input type (a bf16 input is exact as bf16) with rows
    // of an odd number of dwords; once the products that read them are done, each
    // region holds a 64 x 64 fp32 matrix (k's: T, q's: A0).  G's region later holds
    // Bk = beta K e^G.  With bf16 inputs this is 67 KB of LDS, so two
    // workgroups share a CU.
    constexpr int KP = H16 ? D + 2 : D + 1;  // elements per staged q or k row
    constexpr int RB = (CH * KP * (int)sizeof(IT) > CH * AP * 4 ? CH * KP * (int)sizeof(IT) : CH * AP * 4);
    __shared__ __align__(16) float sG[CH * DP];
    __shared__ __align__(16) unsigned char sKT[RB];
    __shared__ __align__(16) unsigned char sQA[RB];
    __shared__ float sB[CH];
    __shared__ float sGL[D];  // G of the chunk's last row
    IT* sK = reinterpret_cast<IT*>(sKT);
    IT* sQ = reinterpret_cast<IT*>(sQA);
    float* sT = reinterpret_cast<float*>(sKT);
    float* sA = reinterpret_cast<float*>(sQA);

    // a.Wc chunks per sequence in this backward window, a.win its index
    const int h = blockIdx.x, s = blockIdx.y / a.Wc, jl = blockIdx.y % a.Wc, j = a.win * a.Wc + jl;
    int64_t tb, L;
    seq_range(a, s, tb, L);
    const int64_t c0 = (int64_t)j * CH;
    if (c0 >= L) return;
    const int n = (int)min<int64_t>(CH, L - c0);
    const int H = a.H;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, li = lane & 15, gq = lane >> 4;
    const IT* q = static_cast<const IT*>(a.q);
    const IT* k = static_cast<const IT*>(a.k);
    float* rec = brec + ((size_t)(s * a.Wc + jl) * H + h) * R::FLOATS;
    _Float16* rec16 = reinterpret_cast<_Float16*>(rec + R::CR);
    // chain operands: P[row][col] (A-row col of dU), Qg[r][c] and -W[r][c] (A-row c of
    // dS), Kh[r][c] (A-row r of dU)
    auto put_p = [&](int row, int col, float x) {
        if constexpr (H16) rec16[C16::at(col >> 4, 0, row, col & 15)] = (_Float16)x;
        else rec[R::CR + C::at(col >> 4, C::ks(row), (col & 15) + 16 * C::kg(row))] = x;
    };
    auto put_qg = [&](int r, int c, float x) {
        if constexpr (H16) rec16[C16::at(C::wave_of(c), C16::fq(C::tile_of(c)), r, c & 15)] = (_Float16)x;
        else rec[R::CR + C::at(C::wave_of(c), C::qbase(c) + C::ks(r), (c & 15) + 16 * C::kg(r))] = x;
    };
    auto put_kh = [&](int r, int c, float x) {
        if constexpr (H16) rec16[C16::at(r >> 4, C16::FKH, c, r & 15)] = (_Float16)x;
        else rec[R::CR + C::at(r >> 4, C::EP + C::ks(c), (r & 15) + 16 * C::kg(c))] = x;
    };
    auto put_mw = [&](int r, int c, float x) {
        if constexpr (H16) rec16[C16::at(C::wave_of(c), C16::fw(C::tile_of(c)), r, c & 15)] = (_Float16)x;
        else rec[R::CR + C::at(C::wave_of(c), C::qbase(c) + C::EQ + C::ks(r), (c & 15) + 16 * C::kg(r))] = x;
    };

    // inputs, branch-free: rows past the sequence end clamped, then zeroed
    constexpr int PER = CH * D / BW_T;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = t + BW_T * i, r = idx / D, c = idx % D;
        const size_t th = (size_t)(tb + c0 + min(r, n - 1)) * H + h;
        const bool ok = r < n;
        const IT kx = k[th * D + c], qx = q[th * D + c];
        const float gx = a.gate_per_head ? a.la[th] : a.la[th * D + c];
        sK[r * KP + c] = ok ? kx : IT{};
        sQ[r * KP + c] = ok ? qx : IT{};
        sG[r * DP + c] = ok ? gx : 0.f;
    }
    if (t < CH) sB[t] = t < n ? a.beta[(size_t)(tb + c0 + t) * H + h] : 0.f;
    __syncthreads();
    if (t < D) {  // inclusive cumulative log-gate per channel, summed in fp64 and rounded once
        double acc = 0.0;
        for (int r = 0; r < CH; ++r) {
            acc += (double)sG[r * DP + t];
            sG[r * DP + t] = (float)acc;
        }
        sGL[t] = sG[(n - 1) * DP + t];
    }
    __syncthreads();
    auto kf = [&](int r, int c) { return to_f32(sK[r * KP + c]); };

    // A0 (strict) and P (inclusive) by 16x16 blocks, anchored: row a for an
    // off-diagonal block (the later block's first row), the block's ninth row
    // for a diagonal one.  P goes to the record; this wave's A0 blocks (tasks
    // wave and wave + BW_W below 10) stay in registers until q's region is free.
    floatx4 a0[2] = {zero4(), zero4()};
    for (int task = wave; task < 20; task += BW_W) {
        const bool isP = task >= 10;
        const int bt = task % 10;
        const int rb = bt < 1 ? 0 : bt < 3 ? 1 : bt < 6 ? 2 : 3;
        const int cb = bt - rb * (rb + 1) / 2;
        const int an = cb < rb ? 16 * rb : 16 * rb + 8;
        const IT* X = isP ? sQ : sK;
        const int rr = 16 * rb + li, ii = 16 * cb + li;
        floatx4 acc = zero4();
        // a diagonal block whose single-anchor exponents pass kWideExp (in either direction:
        // the block's first row over the anchor, the anchor over its last row) is formed in
        // the multi-level form instead
        bool wide = false;
        if (cb == rb) {
            float ex = 0.f;
            for (int c = lane; c < D; c += 64)
                ex = fmaxf(ex, fmaxf(sG[(16 * rb) * DP + c] - sG[an * DP + c], sG[an * DP + c] - sG[(16 * rb + 15) * DP + c]));
            wide = __any(!(ex <= kWideExp));
        }
        if (!wide) {
            tile_f32(acc, D, lane,
                     [&](int c) { return to_f32(X[rr * KP + c]) * fast_exp(sG[rr * DP + c] - sG[an * DP + c]); },
                     [&](int c) { return kf(ii, c) * fast_exp(sG[an * DP + c] - sG[ii * DP + c]); });
        } else {
            // level lev: pairs (r, i) in the later / earlier half of an aligned sub-block of
            // sz rows, anchored at its middle row; a last level (isP only) for the diagonal
            for (int lev = 0; lev < (isP ? 5 : 4); ++lev) {
                const bool dg = lev == 4;
                const int sz = dg ? 1 : 16 >> lev, hs = sz >> 1, msk = sz - 1;
                const int ra = 16 * rb + (li & ~msk) + hs;  // anchor of row li / column li
                floatx4 lv = zero4();
                tile_f32(lv, D, lane,
                         [&](int c) {
                             const float x = to_f32(X[rr * KP + c]);
                             return dg ? x
                                       : ((li & msk) >= hs ? x * fast_exp(sG[rr * DP + c] - sG[ra * DP + c]) : 0.f);
                         },
                         [&](int c) {
                             const float x = kf(ii, c);
                             return dg ? x : ((li & msk) < hs ? x * fast_exp(sG[ra * DP + c] - sG[ii * DP + c]) : 0.f);
                         });
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lr = 4 * gq + r;
                    const bool pair = dg ? lr == li
                                         : (lr & ~msk) == (li & ~msk) && (lr & msk) >= hs && (li & msk) < hs;
                    if (pair) acc[r] = lv[r];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rb + 4 * gq + r, col = 16 * cb + li;
            const bool keep = cb < rb || (isP ? row >= col : row > col);
            const float x = keep ? acc[r] : 0.f;
            if (isP) put_p(row, col, x);
            else if (task < BW_W) a0[0][r] = x;
            else a0[1][r] = x;
        }
    }
    // P's upper blocks in the record
    for (int idx = t; idx < CH * CH; idx += BW_T) {
        const int r = idx / CH, c = idx % CH;
        if ((c >> 4) > (r >> 4)) put_p(r, c, 0.f);
    }
    __syncthreads();
    // Qg, Kh, G and gamma to the record; Bk = beta K e^G replaces G in LDS (each
    // element by the thread that read it)
    for (int idx = t; idx < CH * D; idx += BW_T) {
        const int r = idx / D, c = idx % D;
        const float g = sG[r * DP + c], e = fast_exp(g), kx = kf(r, c);
        put_qg(r, c, to_f32(sQ[r * KP + c]) * e);
        put_kh(r, c, kx * fast_exp(sGL[c] - g));
        rec[R::G + idx] = g;
        sG[r * DP + c] = sB[r] * kx * e;
    }
    __syncthreads();
    // q and k are no longer read: A0 into q's region (this wave's blocks, then zero
    // upper blocks), T zeroed in k's
    for (int task = wave, i = 0; task < 10; task += BW_W, ++i) {
        const int rb = task < 1 ? 0 : task < 3 ? 1 : task < 6 ? 2 : 3;
        const int cb = task - rb * (rb + 1) / 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) sA[(16 * rb + 4 * gq + r) * AP + 16 * cb + li] = a0[i][r];
    }
    for (int idx = t; idx < CH * CH; idx += BW_T) {
        const int r = idx / CH, c = idx % CH;
        if ((c >> 4) > (r >> 4)) sA[r * AP + c] = 0.f;
        sT[r * AP + c] = 0.f;
    }
    __syncthreads();
    for (int idx = t; idx < CH * CH; idx += BW_T) {  // A0 to the record, then Atil = diag(beta) A0 in LDS
        const int r = idx / CH, c = idx % CH;
        rec[R::A0 + idx] = sA[r * AP + c];
        sA[r * AP + c] *= sB[r];
    }
    __syncthreads();
    // T = (I + Atil)^-1 (the same product form and block inversion as the forward's)
    ut_inverse64<AP, BW_W>(sT, sA, wave, lane);
    for (int idx = t; idx < CH * CH; idx += BW_T) {  // the scratch blocks above the diagonal read as zero
        const int r = idx / CH, c = idx % CH;
        if ((c >> 4) > (r >> 4)) sT[r * AP + c] = 0.f;
    }
    __syncthreads();
    for (int idx = t; idx < CH * CH; idx += BW_T) rec[R::T + idx] = sT[(idx / CH) * AP + idx % CH];
    const float* GL = sGL;
    for (int idx = t; idx < D * 16; idx += BW_T) {  // gamma of dS row c, for every li
        const int c = idx / 16, l = (idx % 16) + 16 * ((c & 15) >> 2);
        if constexpr (H16) rec[R::CR + C16::gam(C::wave_of(c), C::tile_of(c), l, c & 3)] = fast_exp(GL[c]);
        else rec[R::CR + ((C::wave_of(c) * C::Q4 + C::E / 4 + C::tile_of(c)) * 64 + l) * 4 + (c & 3)] = fast_exp(GL[c]);
    }
    __syncthreads();
    for (int task = wave; task < 4 * (D / 16); task += BW_W) {
        const int mt = task / (D / 16), nt = task % (D / 16);
        const int cc = 16 * nt + li;
        floatx4 acc = zero4();
        // T is lower triangular: row block mt sees columns below 16 (mt + 1)
        tile_f32(acc, 16 * (mt + 1), lane, [&](int i) { return sT[(16 * mt + li) * AP + i]; },
                 [&](int i) { return sG[i * DP + cc]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) put_mw(16 * mt + 4 * gq + r, cc, -acc[r]);
    }
}

// ---------------------------------------------------------------------------
// reverse chain over the chunks of one (sequence, head), 16 value columns
// ---------------------------------------------------------------------------
// Each wave's operands for chunk j - 1 (its slice of the chain record, one
// float4 per four matrix-core steps) and the next dO slice are loaded into
// registers while chunk j is computed, so the serial chain waits on the
// matrix cores and two barriers per chunk, not on memory.
// Chunks a.win * a.Wc .. of each sequence (one backward window), from the last
// to the first: dS starts as dS_in (dL/dS at the window's end; null: zero) and
// its value entering the window goes to dS_out (null: not stored).  dS_in and
// dS_out may be the same array: each workgroup reads and writes only its own
// slice.
template <int D, typename GT>
__global__ void __launch_bounds__(256) bwd_chain_kernel(ChunkArgs a, const float* brec, const GT* dO,
                                                        const float* dS_in, float* dsnap, float* dU, float* dS_out) {
    using R = BRec<D>;
    using C = ChainRec<D>;
    // B operands transposed: column li of the slice, reduction index contiguous
    constexpr int KS = D + 4, KO = CH + 4;
    constexpr int DO_PER = CH * 16 / 256;  // dO values per thread and chunk
    __shared__ __align__(16) float sdS[16 * KS];
    __shared__ __align__(16) float sdO[2][16 * KO];
    __shared__ __align__(16) float sdU[16 * KO];
    const int H = a.H, NH = a.N * H;
    const int u = blockIdx.x % NH, z = blockIdx.x / NH;
    const int s = u / H, h = u % H, col0 = 16 * z;
    int64_t tb, L;
    seq_range(a, s, tb, L);
    const int j0 = a.win * a.Wc;
    const int nch = (int)min<int64_t>((L + CH - 1) / CH, (int64_t)j0 + a.Wc);  // one past the window's last chunk
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, li = lane & 15, gq = lane >> 4;
    auto crec = [&](int j) {
        return reinterpret_cast<const float4*>(brec + ((size_t)(s * a.Wc + (j - j0)) * H + h) * R::FLOATS + R::CR) +
               (size_t)wave * C::Q4 * 64 + lane;
    };
    // dO of chunk j: thread t holds rows (t + 256 i) / 16, clamped to the sequence;
    // rows past its end are zeroed when stored to LDS, so the loads stay in flight
    auto rows = [&](int j) { return (int)min<int64_t>(CH, L - (int64_t)j * CH); };
    auto load_do = [&](int j, GT* x) {
        const int n = rows(j);
#pragma unroll
        for (int i = 0; i < DO_PER; ++i) {
            const int idx = t + 256 * i, r = idx / 16, vv = idx % 16;
            x[i] = dO[((size_t)(tb + (int64_t)j * CH + min(r, n - 1)) * H + h) * D + col0 + vv];
        }
    };
    auto store_do = [&](int buf, int j, const GT* x) {
        const int n = rows(j);
#pragma unroll
        for (int i = 0; i < DO_PER; ++i) {
            const int idx = t + 256 * i, r = idx / 16;
            sdO[buf][(idx % 16) * KO + r] = r < n ? to_f32(x[i]) : 0.f;
        }
    };
    float4 cur[C::Q4], nxt[C::Q4];
    GT don[DO_PER];
    if (nch > j0) {
        const float4* p = crec(nch - 1);
#pragma unroll
        for (int i = 0; i < C::Q4; ++i) cur[i] = p[i * 64];
        load_do(nch - 1, don);
        store_do(0, nch - 1, don);
    }
    auto mfma4 = [](floatx4 acc, float4 x, float4 y) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, y.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, y.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, y.z, acc, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, y.w, acc, 0, 0, 0);
    };
    for (int idx = t; idx < D * 16; idx += 256) {
        const int c = idx / 16, vv = idx % 16;
        sdS[vv * KS + c] = dS_in ? dS_in[((size_t)u * D + c) * D + col0 + vv] : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < nch - j0; ++jj) {
        const int j = nch - 1 - jj, buf = jj & 1;
        if (j > j0) {
            load_do(j - 1, don);
            const float4* p = crec(j - 1);
#pragma unroll
            for (int i = 0; i < C::Q4; ++i) nxt[i] = p[i * 64];
        }
        const size_t ch = (size_t)(s * a.Wc + (j - j0)) * H + h;
        float* snap = dsnap + ch * D * D;
#pragma unroll
        for (int i = 0; i < D * 4 / 256; ++i) {  // dL/dS_{j+1}, four columns per store
            const int idx = t + 256 * i, c = idx / 4, v4 = 4 * (idx % 4);
            *reinterpret_cast<float4*>(snap + (size_t)c * D + col0 + v4) =
                make_float4(sdS[v4 * KS + c], sdS[(v4 + 1) * KS + c], sdS[(v4 + 2) * KS + c], sdS[(v4 + 3) * KS + c]);
        }
        const float* sO = sdO[buf] + li * KO + 4 * gq;
        const float* sS = sdS + li * KS + 4 * gq;
        {  // dU = P^T dO + Kh dS: rows 16 wave .. 16 wave + 15
            floatx4 acc = zero4();
#pragma unroll
            for (int b = 0; b < C::EP / 4; ++b) acc = mfma4(acc, cur[b], lds4(sO + 16 * b));
#pragma unroll
            for (int b = 0; b < C::EK / 4; ++b) acc = mfma4(acc, cur[C::EP / 4 + b], lds4(sS + 16 * b));
            *reinterpret_cast<float4*>(sdU + li * KO + 16 * wave + 4 * gq) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            float* du = dU + ch * CH * D;
#pragma unroll
            for (int r = 0; r < 4; ++r) du[(size_t)(16 * wave + 4 * gq + r) * D + col0 + li] = acc[r];
        }
        lds_barrier();  // orders LDS only: the next chunk's loads stay in flight
        // dS <- Diag(gamma) dS + Qg^T dO - W^T dU: tiles at rows wave D/4 + 16 rt
        const float* sU = sdU + li * KO + 4 * gq;
#pragma unroll
        for (int rt = 0; rt < C::NRT; ++rt) {
            const int cb = wave * (D / 4) + 16 * rt, qb = (C::EP + C::EK + rt * 2 * C::EQ) / 4;
            const float4 gm = cur[C::E / 4 + rt], s4 = lds4(sS + cb);
            floatx4 acc;
            acc[0] = gm.x * s4.x;
            acc[1] = gm.y * s4.y;
            acc[2] = gm.z * s4.z;
            acc[3] = gm.w * s4.w;
#pragma unroll
            for (int b = 0; b < C::EQ / 4; ++b) acc = mfma4(acc, cur[qb + b], lds4(sO + 16 * b));
#pragma unroll
            for (int b = 0; b < C::EQ / 4; ++b) acc = mfma4(acc, cur[qb + C::EQ / 4 + b], lds4(sU + 16 * b));
            *reinterpret_cast<float4*>(sdS + li * KS + cb + 4 * gq) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        if (j > j0) store_do(buf ^ 1, j - 1, don);
        lds_barrier();  // orders LDS only: the next chunk's loads stay in flight
        if (j > j0) {
#pragma unroll
            for (int i = 0; i < C::Q4; ++i) cur[i] = nxt[i];
        }
    }
    if (dS_out)
        for (int idx = t; idx < D * 16; idx += 256) {
            const int c = idx / 16, vv = idx % 16;
            dS_out[((size_t)u * D + c) * D + col0 + vv] = sdS[vv * KS + c];
        }
}

// four fp32 values as four adjacent fp16 operand elements
__device__ __forceinline__ void put_h4(_Float16* dst, floatx4 x) {
    half4 h;
    h[0] = (_Float16)x[0];
    h[1] = (_Float16)x[1];
    h[2] = (_Float16)x[2];
    h[3] = (_Float16)x[3];
    *reinterpret_cast<half4*>(dst) = h;
}

// The reverse chain with fp16 matrix-core operands (bf16 inputs): the same
// steps as bwd_chain_kernel, each wave's operands as ChainRec16 fragments and
// the B operands dO^T, dS^T and dU^T as fp16 rows in LDS.  dS itself stays in
// fp32 (the Diag(gamma) term, the stored gradient snapshots and the carried
// value); only its copy used as an operand is rounded.
template <int D, typename GT>
__global__ void __launch_bounds__(256) bwd_chain16_kernel(ChunkArgs a, const float* brec, const GT* dO,
                                                          const float* dS_in, float* dsnap, float* dU,
                                                          float* dS_out) {
    using R = BRec<D>;
    using C = ChainRec16<D>;
    constexpr int KS = D + 4;             // fp32 dS^T rows
    constexpr int SP = D + 8, OP = CH + 8;  // fp16 operand rows (16-byte aligned, staggered banks)
    constexpr int DO_PER = CH * 16 / 256;
    __shared__ __align__(16) float sdS[16 * KS];
    __shared__ __align__(16) _Float16 sS16[16 * SP];
    __shared__ __align__(16) _Float16 sO16[2][16 * OP];
    __shared__ __align__(16) _Float16 sU16[16 * OP];
    const int H = a.H, NH = a.N * H;
    const int u = blockIdx.x % NH, z = blockIdx.x / NH;
    const int s = u / H, h = u % H, col0 = 16 * z;
    int64_t tb, L;
    seq_range(a, s, tb, L);
    const int j0 = a.win * a.Wc;
    const int nch = (int)min<int64_t>((L + CH - 1) / CH, (int64_t)j0 + a.Wc);  // one past the window's last chunk
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, li = lane & 15, gq = lane >> 4;
    auto crec = [&](int j) { return brec + ((size_t)(s * a.Wc + (j - j0)) * H + h) * R::FLOATS + R::CR; };
    auto load_ops = [&](int j, half8* f, float4* g) {
        const float* p = crec(j);
        const half8* pf = reinterpret_cast<const half8*>(p) + (size_t)wave * C::F * 64 + lane;
#pragma unroll
        for (int i = 0; i < C::F; ++i) f[i] = pf[i * 64];
#pragma unroll
        for (int rt = 0; rt < C::NRT; ++rt) g[rt] = *reinterpret_cast<const float4*>(p + C::gam(wave, rt, lane, 0));
    };
    auto rows = [&](int j) { return (int)min<int64_t>(CH, L - (int64_t)j * CH); };
    auto load_do = [&](int j, GT* x) {
        const int n = rows(j);
#pragma unroll
        for (int i = 0; i < DO_PER; ++i) {
            const int idx = t + 256 * i, r = idx / 16, vv = idx % 16;
            x[i] = dO[((size_t)(tb + (int64_t)j * CH + min(r, n - 1)) * H + h) * D + col0 + vv];
        }
    };
    auto store_do = [&](int buf, int j, const GT* x) {
        const int n = rows(j);
#pragma unroll
        for (int i = 0; i < DO_PER; ++i) {
            const int idx = t + 256 * i, r = idx / 16;
            sO16[buf][(idx % 16) * OP + r] = (_Float16)(r < n ? to_f32(x[i]) : 0.f);
        }
    };
    auto mfma = [](half8 x, const _Float16* y, floatx4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, *reinterpret_cast<const half8*>(y), acc, 0, 0, 0);
    };
    // operands of three chunks in flight: chunk j is computed from buffer p while
    // chunk j - 2 is loaded into buffer p + 2 (mod 3); the loop is unrolled by three
    // so the buffers rotate by name and no register copy waits on a load
    half8 ops[3][C::F];
    float4 gam[3][C::NRT];
    GT dob[3][DO_PER];
    if (nch > j0) {
        load_ops(nch - 1, ops[0], gam[0]);
        load_do(nch - 1, dob[0]);
        store_do(0, nch - 1, dob[0]);
        if (nch - 2 >= j0) {
            load_ops(nch - 2, ops[1], gam[1]);
            load_do(nch - 2, dob[1]);
        }
    }
    for (int idx = t; idx < D * 16; idx += 256) {
        const int c = idx / 16, vv = idx % 16;
        const float x = dS_in ? dS_in[((size_t)u * D + c) * D + col0 + vv] : 0.f;
        sdS[vv * KS + c] = x;
        sS16[vv * SP + c] = (_Float16)x;
    }
    __syncthreads();
    for (int jj0 = 0; jj0 < nch - j0; jj0 += 3) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            const int jj = jj0 + p, j = nch - 1 - jj, buf = jj & 1;
            if (j < j0) break;
            const half8* cur = ops[p];
            if (j - 2 >= j0) {
                load_ops(j - 2, ops[(p + 2) % 3], gam[(p + 2) % 3]);
                load_do(j - 2, dob[(p + 2) % 3]);
            }
            const size_t ch = (size_t)(s * a.Wc + (j - j0)) * H + h;
            float* snap = dsnap + ch * D * D;
#pragma unroll
            for (int i = 0; i < D * 4 / 256; ++i) {  // dL/dS_{j+1}, four columns per store
                const int idx = t + 256 * i, c = idx / 4, v4 = 4 * (idx % 4);
                *reinterpret_cast<float4*>(snap + (size_t)c * D + col0 + v4) = make_float4(
                    sdS[v4 * KS + c], sdS[(v4 + 1) * KS + c], sdS[(v4 + 2) * KS + c], sdS[(v4 + 3) * KS + c]);
            }
            const _Float16* bO = sO16[buf] + li * OP + 8 * gq;
            const _Float16* bS = sS16 + li * SP + 8 * gq;
            {  // dU = P^T dO + Kh dS: rows 16 wave .. 16 wave + 15
                floatx4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) acc = mfma(cur[kk], bO + 32 * kk, acc);
#pragma unroll
                for (int kk = 0; kk < C::FK; ++kk) acc = mfma(cur[C::FKH + kk], bS + 32 * kk, acc);
                put_h4(sU16 + li * OP + 16 * wave + 4 * gq, acc);
                float* du = dU + ch * CH * D;
#pragma unroll
                for (int r = 0; r < 4; ++r) du[(size_t)(16 * wave + 4 * gq + r) * D + col0 + li] = acc[r];
            }
            lds_barrier();  // orders LDS only: the later chunks' loads stay in flight
            // dS <- Diag(gamma) dS + Qg^T dO - W^T dU: tiles at rows wave D/4 + 16 rt
            const _Float16* bU = sU16 + li * OP + 8 * gq;
#pragma unroll
            for (int rt = 0; rt < C::NRT; ++rt) {
                const int cb = wave * (D / 4) + 16 * rt;
                const float4 gm = gam[p][rt], s4 = *reinterpret_cast<const float4*>(sdS + li * KS + cb + 4 * gq);
                floatx4 acc;
                acc[0] = gm.x * s4.x;
                acc[1] = gm.y * s4.y;
                acc[2] = gm.z * s4.z;
                acc[3] = gm.w * s4.w;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) acc = mfma(cur[C::fq(rt) + kk], bO + 32 * kk, acc);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) acc = mfma(cur[C::fw(rt) + kk], bU + 32 * kk, acc);
                *reinterpret_cast<float4*>(sdS + li * KS + cb + 4 * gq) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                put_h4(sS16 + li * SP + cb + 4 * gq, acc);
            }
            if (j > j0) store_do(buf ^ 1, j - 1, dob[(p + 1) % 3]);
            lds_barrier();
        }
    }
    if (dS_out)
        for (int idx = t; idx < D * 16; idx += 256) {
            const int c = idx / 16, vv = idx % 16;
            dS_out[((size_t)u * D + c) * D + col0 + vv] = sdS[vv * KS + c];
        }
}

// ---------------------------------------------------------------------------
// local: every parameter gradient of one (chunk, head)
// ---------------------------------------------------------------------------
// Eight waves; wave w owns the 16x16 tiles w, w + 8, ... of every 64 x D
// gradient and keeps dq, dk and the k-part of dG for them in registers across
// all products: every dq contribution carries dG += q o dq and every dk
// contribution dG += +-k o dk, so dG = q o dq + k o (signed dk part) needs no
// pass over memory.  Inputs are read branch-free (rows past the sequence end
// clamped, then zeroed).
template <int D, typename IT, typename GT>
__global__ void __launch_bounds__(BL_T) bwd_local_kernel(BwdArgs b) {
    const ChunkArgs& a = b.fwd;
    const float* brec = b.brec;
    const GT* dO = static_cast<const GT*>(b.dO);
    using R = BRec<D>;
    constexpr int DP = D + 4;
    constexpr int GD = D + 4;
    constexpr int AP = CH + 1;
    constexpr int NB = D / 16;            // 16-column blocks of a 64 x D matrix
    constexpr int TPW = 4 * NB / BL_W;    // tiles of such a matrix per wave
    __shared__ __align__(16) float sG[CH * GD];  // G, rows padded against bank conflicts
    __shared__ float sT[CH * AP];
    __shared__ __align__(16) float sX[CH * DP];   // U, dW, dU, T^T dT, q, dG
    __shared__ __align__(16) float sY[CH * DP];   // dO, Bk, Bv, k
    __shared__ float sP[CH * AP];   // dP, then column partial sums
    __shared__ float sM[CH * AP];   // dT, then diag(beta) dAtil
    __shared__ float sGL[D];        // dL/dG_last per channel
    __shared__ float sdB[CH];
    __shared__ float sdBw[BL_W][CH];  // each wave's dBk and dBv part of dbeta, per row
    __shared__ float sBeta[CH];

    const int h = blockIdx.x, s = blockIdx.y / a.Wc, jl = blockIdx.y % a.Wc, j = a.win * a.Wc + jl;
    int64_t tb, L;
    seq_range(a, s, tb, L);
    const int64_t c0 = (int64_t)j * CH;
    if (c0 >= L) return;
    const int n = (int)min<int64_t>(CH, L - c0);
    const int H = a.H;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, li = lane & 15, gq = lane >> 4;
    const IT* q = static_cast<const IT*>(a.q);
    const IT* k = static_cast<const IT*>(a.k);
    const IT* v = static_cast<const IT*>(a.v);
    const size_t ch = (size_t)(s * a.Wc + jl) * H + h;
    const float* rec = brec + ch * R::FLOATS;
    const float* S = a.snap + ch * D * D;
    const float* dS = b.dsnap + ch * D * D;
    const float* dU = b.dU + ch * CH * D;
    // row r of a [T, H, D] tensor, clamped to the chunk's last row
    auto tok = [&](int r) { return ((size_t)(tb + c0 + min(r, n - 1)) * H + h) * D; };
    auto in = [&](const IT* p, int r, int c) {
        const float x = ld(p, tok(r) + c);
        return r < n ? x : 0.f;
    };
    auto mt_of = [&](int i) { return (wave + BL_W * i) / NB; };
    auto nt_of = [&](int i) { return (wave + BL_W * i) % NB; };
    floatx4 aq[TPW], ak[TPW], aks[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) aq[i] = ak[i] = aks[i] = zero4();

    // copies to LDS: every thread's loads are issued before its stores
    constexpr int V4 = CH * D / 4 / BL_T;  // float4s of a 64 x D matrix per thread
    {
        float4 g[V4], tt[CH * CH / 4 / BL_T];
#pragma unroll
        for (int i = 0; i < V4; ++i) g[i] = ld4(rec + R::G, 4 * (t + BL_T * i));
#pragma unroll
        for (int i = 0; i < CH * CH / 4 / BL_T; ++i) tt[i] = ld4(rec + R::T, 4 * (t + BL_T * i));
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int idx = 4 * (t + BL_T * i);
            *reinterpret_cast<float4*>(sG + (idx / D) * GD + idx % D) = g[i];
        }
#pragma unroll
        for (int i = 0; i < CH * CH / 4 / BL_T; ++i) {
            const int idx = 4 * (t + BL_T * i), r = idx / CH, c = idx % CH;
            sT[r * AP + c] = tt[i].x;
            sT[r * AP + c + 1] = tt[i].y;
            sT[r * AP + c + 2] = tt[i].z;
            sT[r * AP + c + 3] = tt[i].w;
        }
    }
    // rows r (clamped, zeroed past the sequence end) of a [T, H, D] tensor to a
    // 64 x D LDS matrix, scaled per element by f(r, c, x)
    auto stage = [&](auto* src, float* dst, auto&& f) {
        float4 x[V4];
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int idx = 4 * (t + BL_T * i), r = idx / D, c = idx % D;
            x[i] = ld4(src, tok(r) + c);
        }
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int idx = 4 * (t + BL_T * i), r = idx / D, c = idx % D;
            const float m = r < n ? 1.f : 0.f;
            float* d = dst + r * DP + c;
            d[0] = f(r, c, m * x[i].x);
            d[1] = f(r, c + 1, m * x[i].y);
            d[2] = f(r, c + 2, m * x[i].z);
            d[3] = f(r, c + 3, m * x[i].w);
        }
    };
    auto same = [](int, int, float x) { return x; };
    if (t < D) sGL[t] = 0.f;
    if (t < CH) {
        sdB[t] = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < BL_W; ++w2) sdBw[w2][t] = 0.f;
        sBeta[t] = t < n ? a.beta[(size_t)(tb + c0 + t) * H + h] : 0.f;
    }
    __syncthreads();
    const float* GL = sG + (n - 1) * GD;

    // U = Ut - W S_j, as the recompute's state pass formed it (rows past the end zeroed)
    {
        float4 x[V4];
#pragma unroll
        for (int i = 0; i < V4; ++i) x[i] = ld4(rec + R::U, 4 * (t + BL_T * i));
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int idx = 4 * (t + BL_T * i), r = idx / D, c = idx % D;
            const float m = r < n ? 1.f : 0.f;
            *reinterpret_cast<float4*>(sX + r * DP + c) = make_float4(m * x[i].x, m * x[i].y, m * x[i].z, m * x[i].w);
        }
    }
    stage(dO, sY, same);
    __syncthreads();
    // dP = tril(dO U^T)
    for (int task = wave; task < 16; task += BL_W) {
        const int mt = task / 4, nt = task % 4;
        floatx4 acc = zero4();
        if (nt <= mt)
            tile_f32_v(acc, D, lane, [&](int c) { return lds4(sY + (16 * mt + li) * DP + c); },
                       [&](int c) { return lds4(sX + (16 * nt + li) * DP + c); });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r, col = 16 * nt + li;
            sP[row * AP + col] = (row >= col && row < n) ? acc[r] : 0.f;
        }
    }
    // dQg = dO S^T -> dq;  dKh = U dS^T -> dk, dG_last (every tile of a wave lies in
    // one 16-column strip, so the wave's dG_last terms add up in registers first)
    // B of both products runs over whole rows of S_j and dS (the strip's channels),
    // which also gives dgamma_c = sum_v S[c][v] dS[c][v] (from one tile per strip)
    float gl = 0.f, dgam = 0.f;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        float dg = 0.f;
        const int mt = mt_of(i), cc = 16 * nt_of(i) + li, rr = 16 * mt + li;
        float kk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) kk[r] = in(k, 16 * mt + 4 * gq + r, cc);
        floatx4 x = zero4(), y = zero4();
        tile2_f32_v<2>(x, y, dg, D, lane, [&](int c) { return lds4(sY + rr * DP + c); },
                       [&](int c) { return ld4(S, (size_t)cc * D + c); }, [&](int c) { return lds4(sX + rr * DP + c); },
                       [&](int c) { return ld4(dS, (size_t)cc * D + c); });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r;
            const float g = sG[row * GD + cc];
            aq[i][r] += x[r] * fast_exp(g);
            const float f = y[r] * fast_exp(GL[cc] - g);
            ak[i][r] += f;
            aks[i][r] -= f;
            gl += f * kk[r];
        }
        if (i == 0) dgam = dg;
    }
    {
        const int c = 16 * nt_of(0) + li;
        dgam += __shfl_xor(dgam, 16);
        dgam += __shfl_xor(dgam, 32);
        // the strip's channels once: the wave holding its first row block
        if (mt_of(0) == 0) gl += gq == 0 ? dgam * fast_exp(GL[c]) : 0.f;
        atomicAdd(&sGL[c], gl);
    }
    __syncthreads();
    // dW = -dU S^T (into sX); Kg = K e^G (into sY; Bk = diag(beta) Kg)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int mt = mt_of(i), cc = 16 * nt_of(i) + li, rr = 16 * mt + li;
        floatx4 acc = zero4();
        tile_f32_v<4>(acc, D, lane, [&](int c) { return ld4(dU, (size_t)rr * D + c); },
                      [&](int c) { return ld4(S, (size_t)cc * D + c); });
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * mt + 4 * gq + r) * DP + cc] = -acc[r];
    }
    stage(k, sY, [&](int r, int c, float x) { return x * fast_exp(sG[r * GD + c]); });
    __syncthreads();
    // dT = tril(dW Bk^T);  dBk = T^T dW -> dk, dbeta
    for (int task = wave; task < 16; task += BL_W) {
        const int mt = task / 4, nt = task % 4;
        floatx4 acc = zero4();
        const float bc = sBeta[16 * nt + li];
        if (nt <= mt)
            tile_f32_v(acc, D, lane, [&](int c) { return lds4(sX + (16 * mt + li) * DP + c); },
                       [&](int c) {
                           const float4 y = lds4(sY + (16 * nt + li) * DP + c);
                           return make_float4(bc * y.x, bc * y.y, bc * y.z, bc * y.w);
                       });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r, col = 16 * nt + li;
            sM[row * AP + col] = row >= col ? acc[r] : 0.f;
        }
    }
    float pb[TPW][4];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int mt = mt_of(i), cc = 16 * nt_of(i) + li, ii = 16 * mt + li;
        floatx4 acc = zero4();
        const int r0 = 16 * mt;  // T[r][ii] = 0 for r < ii: rows from the tile's own block
        tile_f32(acc, CH - r0, lane, [&](int r) { return sT[(r0 + r) * AP + ii]; },
                 [&](int r) { return sX[(r0 + r) * DP + cc]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r;
            const float dkc = sBeta[row] * fast_exp(sG[row * GD + cc]) * acc[r];
            ak[i][r] += dkc;
            aks[i][r] += dkc;
            pb[i][r] = acc[r] * sY[row * DP + cc];  // with dBv's below: this lane's column of dbeta
        }
    }
    __syncthreads();
    // dU to LDS (sX: dW's last reader, dBk, is done), beside V
    {
        float4 x[V4];
#pragma unroll
        for (int i = 0; i < V4; ++i) x[i] = ld4(dU, 4 * (t + BL_T * i));
        stage(v, sY, same);
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int idx = 4 * (t + BL_T * i);
            *reinterpret_cast<float4*>(sX + (idx / D) * DP + idx % D) = x[i];
        }
    }
    __syncthreads();
    // dT += tril(dU Bv^T) (the same tasks per wave as above, Bv = diag(beta) V);  dBv = T^T dU -> dv, dbeta
    for (int task = wave; task < 16; task += BL_W) {
        const int mt = task / 4, nt = task % 4;
        if (nt > mt) continue;
        floatx4 acc = zero4();
        const float bc = sBeta[16 * nt + li];
        tile_f32_v<4>(acc, D, lane, [&](int c) { return lds4(sX + (16 * mt + li) * DP + c); },
                      [&](int c) {
                          const float4 y = lds4(sY + (16 * nt + li) * DP + c);
                          return make_float4(bc * y.x, bc * y.y, bc * y.z, bc * y.w);
                      });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r, col = 16 * nt + li;
            if (row >= col) sM[row * AP + col] += acc[r];
        }
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int mt = mt_of(i), cc = 16 * nt_of(i) + li, ii = 16 * mt + li;
        floatx4 acc = zero4();
        const int r0 = 16 * mt;
        tile_f32(acc, CH - r0, lane, [&](int r) { return sT[(r0 + r) * AP + ii]; },
                 [&](int r) { return sX[(r0 + r) * DP + cc]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r;
            if (row < n) b.dv[tok(row) + cc] = sBeta[row] * acc[r];
            pb[i][r] += acc[r] * sY[row * DP + cc];
        }
    }
    // this wave's 16 columns of every row it holds: a row sum over the lanes, one
    // writer per row (no two waves write one entry)
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = row16_sum(pb[i][r]);
            if (li == 0) sdBw[wave][16 * mt_of(i) + 4 * gq + r] = x;
        }
    __syncthreads();
    // X = T^T dT (into sX as 64 x 64), then dAtil = -X T^T (strictly lower, into sM)
    for (int task = wave; task < 16; task += BL_W) {
        const int mt = task / 4, nt = task % 4;
        floatx4 acc = zero4();
        const int r0 = 16 * max(mt, nt);  // T^T is upper and dT lower triangular
        tile_f32(acc, CH - r0, lane, [&](int r) { return sT[(r0 + r) * AP + 16 * mt + li]; },
                 [&](int r) { return sM[(r0 + r) * AP + 16 * nt + li]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * mt + 4 * gq + r) * DP + 16 * nt + li] = acc[r];
    }
    __syncthreads();
    for (int task = wave; task < 16; task += BL_W) {
        const int mt = task / 4, nt = task % 4;
        floatx4 acc = zero4();
        if (nt <= mt)  // strictly lower result; T^T is upper triangular: columns below 16 (nt + 1)
            tile_f32(acc, 16 * (nt + 1), lane, [&](int jj) { return sX[(16 * mt + li) * DP + jj]; },
                     [&](int jj) { return sT[(16 * nt + li) * AP + jj]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r, col = 16 * nt + li;
            sM[row * AP + col] = (row > col && row < n) ? -acc[r] : 0.f;
        }
    }
    __syncthreads();
    // dbeta += sum_i dAtil[r][i] A0[r][i];  then sM <- diag(beta) dAtil;  q, k to LDS
    {
        float a0[CH / BL_W];
#pragma unroll
        for (int i = 0; i < CH / BL_W; ++i) a0[i] = rec[R::A0 + (wave + BL_W * i) * CH + lane];
#pragma unroll
        for (int i = 0; i < CH / BL_W; ++i) {
            const int r = wave + BL_W * i;
            float x = sM[r * AP + lane] * a0[i];
            for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
            if (lane == 0) sdB[r] += x;
            sM[r * AP + lane] *= sBeta[r];
        }
    }
    stage(q, sX, same);
    stage(k, sY, same);
    __syncthreads();

    // Decay-weighted products of a lower-triangular M (dP or diag(beta) dAtil):
    //   row form  Y[r][c] = sum_i M[r][i] X[i][c] e^{G_rc - G_ic}
    //   col form  Z[i][c] = sum_r M[r][i] X[r][c] e^{G_rc - G_ic}
    // per tile of the wave and form, the off-diagonal blocks anchored at the
    // block boundary, the diagonal block at its ninth row (or level by level,
    // as in the prep kernel, when that anchor's exponents pass kWideExp).
    //   R1 = row(dP, K) -> dq     C1 = col(dP, Q) -> dk, -k dG
    //   R2 = row(M2, K) -> dk, +k dG     C2 = col(M2, K) -> dk, -k dG
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int blk = mt_of(i), cc = 16 * nt_of(i) + li;
        const int m = 16 * blk + 8;
        const bool wide = __any(!(fmaxf(sG[(16 * blk) * GD + cc] - sG[m * GD + cc],
                                        sG[m * GD + cc] - sG[(16 * blk + 15) * GD + cc]) <= kWideExp));
#pragma unroll 1
        for (int form = 0; form < 4; ++form) {
            const float* M = form < 2 ? sP : sM;
            const float* X = form == 1 ? sX : sY;
            const bool col = form == 1 || form == 3;
            floatx4 off = zero4(), dia = zero4();
            if (!col) {
                const int an = 16 * blk, mr = 16 * blk + li;
                if (blk > 0)
                    tile_f32(off, an, lane, [&](int ii) { return M[mr * AP + ii]; },
                             [&](int ii) { return X[ii * DP + cc] * fast_exp(sG[an * GD + cc] - sG[ii * GD + cc]); });
                if (!wide)
                    tile_f32(dia, 16, lane, [&](int ii) { return M[mr * AP + 16 * blk + ii]; },
                             [&](int ii) {
                                 const int i2 = 16 * blk + ii;
                                 return X[i2 * DP + cc] * fast_exp(sG[m * GD + cc] - sG[i2 * GD + cc]);
                             });
            } else {
                const int bn = 16 * blk + 15, mi = 16 * blk + li;
                if (blk < 3)
                    tile_f32(off, CH - 16 * (blk + 1), lane, [&](int r) { return M[(bn + 1 + r) * AP + mi]; },
                             [&](int r) {
                                 const int rr = bn + 1 + r;
                                 return X[rr * DP + cc] * fast_exp(sG[rr * GD + cc] - sG[bn * GD + cc]);
                             });
                if (!wide)
                    tile_f32(dia, 16, lane, [&](int r) { return M[(16 * blk + r) * AP + mi]; },
                             [&](int r) {
                                 const int rr = 16 * blk + r;
                                 return X[rr * DP + cc] * fast_exp(sG[rr * GD + cc] - sG[m * GD + cc]);
                             });
            }
            if (wide) {
                // the diagonal block level by level, each level's factors applied in full
                // (dia then holds the finished contribution of the block), plus M's diagonal
                const int b0 = 16 * blk;
                for (int lev = 0; lev < 4; ++lev) {
                    const int sz = 16 >> lev, hs = sz >> 1, msk = sz - 1;
                    auto pair = [&](int r, int c) {
                        return (r & ~msk) == (c & ~msk) && (r & msk) >= hs && (c & msk) < hs;
                    };
                    auto anc = [&](int x) { return b0 + (x & ~msk) + hs; };  // anchor of local row x
                    floatx4 lv = zero4();
                    if (!col) {
                        tile_f32(lv, 16, lane, [&](int k) { return pair(li, k) ? M[(b0 + li) * AP + b0 + k] : 0.f; },
                                 [&](int k) {
                                     return (k & msk) < hs
                                                ? X[(b0 + k) * DP + cc] * fast_exp(sG[anc(k) * GD + cc] - sG[(b0 + k) * GD + cc])
                                                : 0.f;
                                 });
                    } else {
                        tile_f32(lv, 16, lane, [&](int k) { return pair(k, li) ? M[(b0 + k) * AP + b0 + li] : 0.f; },
                                 [&](int k) {
                                     return (k & msk) >= hs
                                                ? X[(b0 + k) * DP + cc] * fast_exp(sG[(b0 + k) * GD + cc] - sG[anc(k) * GD + cc])
                                                : 0.f;
                                 });
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int x = 4 * gq + r;  // output row (row form) or column (col form) of the block
                        const bool keep = col ? (x & msk) < hs : (x & msk) >= hs;
                        const float f = col ? fast_exp(sG[anc(x) * GD + cc] - sG[(b0 + x) * GD + cc])
                                            : fast_exp(sG[(b0 + x) * GD + cc] - sG[anc(x) * GD + cc]);
                        dia[r] += keep ? lv[r] * f : 0.f;
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = b0 + 4 * gq + r;
                    dia[r] += M[row * AP + row] * X[row * DP + cc];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * blk + 4 * gq + r;
                const float g = sG[row * GD + cc];
                float y;
                if (!col) {
                    y = wide ? dia[r] : dia[r] * fast_exp(g - sG[m * GD + cc]);
                    if (blk > 0) y += off[r] * fast_exp(g - sG[16 * blk * GD + cc]);
                } else {
                    y = wide ? dia[r] : dia[r] * fast_exp(sG[m * GD + cc] - g);
                    if (blk < 3) y += off[r] * fast_exp(sG[(16 * blk + 15) * GD + cc] - g);
                }
                if (form == 0) {
                    aq[i][r] += y;
                } else {
                    ak[i][r] += y;
                    aks[i][r] += form == 2 ? y : -y;
                }
            }
        }
    }
    // dq, dk out; dG = q o dq + k o (signed dk part)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int mt = mt_of(i), cc = 16 * nt_of(i) + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r;
            aks[i][r] = sX[row * DP + cc] * aq[i][r] + sY[row * DP + cc] * aks[i][r];
            if (row < n) {
                b.dq[tok(row) + cc] = aq[i][r];
                b.dk[tok(row) + cc] = ak[i][r];
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int mt = mt_of(i), cc = 16 * nt_of(i) + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * mt + 4 * gq + r) * DP + cc] = aks[i][r];
    }
    __syncthreads();
    // dlog_alpha = reverse cumulative sum of dG down the chunk's rows, dG_last
    // entering at the last row: column c, row range part of PARTS
    constexpr int PARTS = BL_T / D, RPP = CH / PARTS;
    const int cg = t % D, part = t / D;
    {
        float x = 0.f;
        for (int r = 0; r < RPP; ++r) x += sX[(part * RPP + r) * DP + cg];
        sP[part * D + cg] = x;
    }
    __syncthreads();
    {
        float carry = sGL[cg];
        for (int p = part + 1; p < PARTS; ++p) carry += sP[p * D + cg];
        for (int r = RPP - 1; r >= 0; --r) {
            const int row = part * RPP + r;
            carry += sX[row * DP + cg];
            if (b.dla_head) sX[row * DP + cg] = carry;
            else if (row < n) b.dG[tok(row) + cg] = carry;
        }
    }
    if (t < n) {
        float x = sdB[t];
#pragma unroll
        for (int w2 = 0; w2 < BL_W; ++w2) x += sdBw[w2][t];
        b.dbeta[(size_t)(tb + c0 + t) * H + h] = x;
    }
    if (b.dla_head) {  // one gate per head: its gradient is the sum over the key channels
        __syncthreads();
        for (int r = wave; r < n; r += BL_W) {
            float x = 0.f;
            for (int c = lane; c < D; c += 64) x += sX[r * DP + c];
            for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
            if (lane == 0) b.dla_head[(size_t)(tb + c0 + r) * H + h] = x;
        }
    }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
size_t bwd_record_bytes(int d) { return (d == 128 ? BRec<128>::FLOATS : BRec<64>::FLOATS) * sizeof(float); }

// Backward windows from the last to the first.  With more than one, a first
// forward pass (no snapshots, no outputs) stores the state entering each later
// window; each window then recomputes its forward records and state snapshots
// from that state, and dL/dS entering it is carried to the next one down.
template <int D, typename IT, typename GT>
static hipError_t bwd_run(const BwdArgs& b, hipStream_t st) {
    const ChunkArgs& a = b.fwd;  // a.Wc: chunks of the longest sequence
    constexpr bool BF = std::is_same<IT, bf16_t>::value;
    const int all = a.Wc, wb = b.bwd_window, rw = b.snap_window;
    const int nbw = (all + wb - 1) / wb;  // backward windows
    const int rpb = (wb + rw - 1) / rw;   // record windows per backward window (exact when nbw > 1)
    const int nrw = (all + rw - 1) / rw;  // record windows over every chunk
    const size_t units = (size_t)a.N * a.H, sb = units * D * D * sizeof(float);
    hipError_t e;
    for (int w = 0; w + 1 < nbw; ++w) {
        if ((e = chunk_snapshot_dispatch(D, BF, a, rw, w * rpb, rpb, false, st, b.f32_records)) != hipSuccess) return e;
        if ((e = hipMemcpyAsync(b.ckpt + (size_t)w * units * D * D, a.state_buf, sb, hipMemcpyDeviceToDevice, st)) !=
            hipSuccess)
            return e;
    }
    for (int w = nbw - 1; w >= 0; --w) {
        if (w > 0 && (e = hipMemcpyAsync(a.state_buf, b.ckpt + (size_t)(w - 1) * units * D * D, sb,
                                         hipMemcpyDeviceToDevice, st)) != hipSuccess)
            return e;
        ChunkArgs r = a;
        r.snap_wc = wb;
        r.snap_j0 = w * wb;
        r.snapU = b.brec + BRec<D>::U;
        r.snapU_stride = BRec<D>::FLOATS;
        if ((e = chunk_snapshot_dispatch(D, BF, r, rw, w * rpb, std::min(rpb, nrw - w * rpb), true, st,
                                         b.f32_records)) != hipSuccess)
            return e;
        BwdArgs bw = b;
        bw.fwd.Wc = wb;
        bw.fwd.win = w;
        const dim3 chunks(a.H, a.N * wb);
        hipLaunchKernelGGL((bwd_prep_kernel<D, IT>), chunks, dim3(BW_T), 0, st, bw.fwd, b.brec);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const float* din = w == nbw - 1 ? b.dfinal : b.dcarry;
        float* dout = w == 0 ? b.dinit : b.dcarry;
        if constexpr (BF)
            hipLaunchKernelGGL((bwd_chain16_kernel<D, GT>), dim3(units * (D / 16)), dim3(256), 0, st, bw.fwd, b.brec,
                               static_cast<const GT*>(b.dO), din, b.dsnap, b.dU, dout);
        else
            hipLaunchKernelGGL((bwd_chain_kernel<D, GT>), dim3(units * (D / 16)), dim3(256), 0, st, bw.fwd, b.brec,
                               static_cast<const GT*>(b.dO), din, b.dsnap, b.dU, dout);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_local_kernel<D, IT, GT>), chunks, dim3(BL_T), 0, st, bw);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t bwd_dispatch(int d, bool in_bf16, bool dout_bf16, const BwdArgs& b, hipStream_t st) {
    if (d == 128) {
        if (in_bf16) return dout_bf16 ? bwd_run<128, bf16_t, bf16_t>(b, st) : bwd_run<128, bf16_t, float>(b, st);
        return dout_bf16 ? bwd_run<128, float, bf16_t>(b, st) : bwd_run<128, float, float>(b, st);
    }
    if (in_bf16) return dout_bf16 ? bwd_run<64, bf16_t, bf16_t>(b, st) : bwd_run<64, bf16_t, float>(b, st);
    return dout_bf16 ? bwd_run<64, float, bf16_t>(b, st) : bwd_run<64, float, float>(b, st);
}

}  // namespace kda
