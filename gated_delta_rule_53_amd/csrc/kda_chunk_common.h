// kda_chunk_common.h -- pieces shared by the chunked prefill kernels (KDA and
// the general DPLR variant): sequence bounds, the record's matrix-core
// fragment order, operand stores, register rows of two channels, the 64x64
// UT inverse and the state pass's output stores and fragment loads.
#pragma once
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

__device__ __forceinline__ void seq_bounds(const ChunkArgs& a, int s, int64_t& t0, int64_t& L) {
    if (a.cu) {
        t0 = a.cu[s];
        L = (int64_t)a.cu[s + 1] - t0;
    } else {
        t0 = (int64_t)s * a.T;
        L = a.T;
    }
}

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Matrix-core fragment order.  The record keeps every A operand of the state
// pass as the sequence of 16 x KS fragments one wave loads: fragment (row tile
// rt, k step kk) is 64 lanes x KE contiguous elements, so each wave load
// instruction reads one contiguous 1 KB block.  Element (r, c) of a matrix
// with NC columns (the contraction dimension) lives at idx(r, c, NC).
template <typename OT>
struct FragOrder {
    static constexpr int KE = sizeof(OT) == 2 ? 8 : 1;  // elements per lane per fragment
    static constexpr int KS = 4 * KE;                   // contraction length of one fragment
    __host__ __device__ static constexpr int idx(int r, int c, int NC) {
        return (((r >> 4) * (NC / KS) + c / KS) * 64 + ((c % KS) / KE) * 16 + (r & 15)) * KE + (c % KE);
    }
    __host__ __device__ static constexpr int frag(int rt, int kk, int lane, int NC) {
        return ((rt * (NC / KS) + kk) * 64 + lane) * KE;
    }
};

template <typename OT>
struct Pad {
    static constexpr int v = sizeof(OT) == 2 ? 8 : 4;  // keeps 16-byte row alignment, breaks bank strides
};

// fp32 tile product with B given row-major (B[k][j] at B + k*ldb + j).
__device__ __forceinline__ void mma_tile_f32_rowB(floatx4& acc, const float* A, int lda, const float* B, int ldb,
                                                  int K, int lane) {
    const int i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[i * lda + k0 + g], B[(k0 + g) * ldb + i], acc, 0, 0, 0);
}

template <typename OT>
__device__ __forceinline__ void store8(OT* dst, const float* x);
template <>
__device__ __forceinline__ void store8<_Float16>(_Float16* dst, const float* x) {
    half8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (_Float16)x[e];
    *reinterpret_cast<half8*>(dst) = a;
}
template <>
__device__ __forceinline__ void store8<float>(float* dst, const float* x) {
    reinterpret_cast<float4*>(dst)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

template <typename OT>
__device__ __forceinline__ void store4(OT* dst, floatx4 x);
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* dst, floatx4 x) {
    half4 h;
    h[0] = (_Float16)x[0];
    h[1] = (_Float16)x[1];
    h[2] = (_Float16)x[2];
    h[3] = (_Float16)x[3];
    *reinterpret_cast<half4*>(dst) = h;
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, floatx4 x) {
    *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
}

template <typename OT>
__device__ __forceinline__ floatx4 load4(const OT* src);
template <>
__device__ __forceinline__ floatx4 load4<_Float16>(const _Float16* src) {
    half4 h = *reinterpret_cast<const half4*>(src);
    floatx4 x = {(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    return x;
}
template <>
__device__ __forceinline__ floatx4 load4<float>(const float* src) {
    float4 v = *reinterpret_cast<const float4*>(src);
    floatx4 x = {v.x, v.y, v.z, v.w};
    return x;
}


// Eight rows of two adjacent channels held in registers: bf16 inputs keep the
// two channels of a row packed in one register (widened exactly on use), fp32
// inputs keep a float2.
template <typename IT>
struct Pair8;
template <>
struct Pair8<bf16_t> {
    uint32_t w[8];
    __device__ __forceinline__ void load(int i, const bf16_t* p) {
        w[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    __device__ __forceinline__ void zero(int i) { w[i] = 0u; }
    __device__ __forceinline__ float get(int i, int e) const {
        return __uint_as_float(e ? (w[i] & 0xFFFF0000u) : (w[i] << 16));
    }
};
template <>
struct Pair8<float> {
    float2 w[8];
    __device__ __forceinline__ void load(int i, const float* p) {
        const float* f = reinterpret_cast<const float*>(p);
        w[i] = make_float2(__builtin_nontemporal_load(f), __builtin_nontemporal_load(f + 1));
    }
    __device__ __forceinline__ void zero(int i) { w[i] = make_float2(0.f, 0.f); }
    __device__ __forceinline__ float get(int i, int e) const { return e ? w[i].y : w[i].x; }
    __device__ __forceinline__ void set(int i, float a, float b) { w[i] = make_float2(a, b); }
};
// L2-normalised bf16 rows: the two channels of a row packed as fp16 (|x| <= 1)
template <>
struct Pair8<_Float16> {
    uint32_t w[8];
    __device__ __forceinline__ void zero(int i) { w[i] = 0u; }
    __device__ __forceinline__ float get(int i, int e) const { return (float)__builtin_bit_cast(half2v, w[i])[e]; }
    __device__ __forceinline__ void set(int i, float a, float b) {
        half2v h;
        h[0] = (_Float16)a;
        h[1] = (_Float16)b;
        w[i] = __builtin_bit_cast(uint32_t, h);
    }
};

// Register type of q and k rows: the input pairs, or fp16 pairs once bf16 rows are normalised.
template <typename IT, bool QKN>
struct QKReg {
    using type = Pair8<IT>;
};
template <>
struct QKReg<bf16_t, true> {
    using type = Pair8<_Float16>;
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f32(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Sum of x over the NP lanes (64 or 32) that hold one row, in every lane: inside
// each 16-lane row through DPP (lane pairs, quads, mirrored half-rows, mirrored
// rows), then across the rows through lane reads -- no LDS traffic.
template <int NP>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f32<0x141>(x);  // row_half_mirror
    x += dpp_f32<0x140>(x);  // row_mirror
    const float a = lane_f32(x, 0), b = lane_f32(x, 16), c = lane_f32(x, 32), d = lane_f32(x, 48);
    if constexpr (NP == 64) {
        return (a + b) + (c + d);
    } else {
        static_assert(NP == 32, "rows span 32 or 64 lanes");
        return (__lane_id() < 32) ? a + b : c + d;
    }
}

// q and k of a thread's eight rows divided by their L2 norms over the key
// channels (the NP lanes that hold a row share its sum of squares).
template <int NP, typename IT, typename QT>
__device__ __forceinline__ void l2norm_rows(const Pair8<IT>& kr, const Pair8<IT>& qr, Pair8<QT>& kk, Pair8<QT>& qq,
                                            float eps) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float k0 = kr.get(i, 0), k1 = kr.get(i, 1), q0 = qr.get(i, 0), q1 = qr.get(i, 1);
        const float sk = row_sum<NP>(k0 * k0 + k1 * k1), sq = row_sum<NP>(q0 * q0 + q1 * q1);
        const float rk = __builtin_amdgcn_rsqf(sk + eps), rq = __builtin_amdgcn_rsqf(sq + eps);
        kk.set(i, k0 * rk, k1 * rk);
        qq.set(i, q0 * rq, q1 * rq);
    }
}

// Two adjacent operand elements of one row.
template <typename OT>
__device__ __forceinline__ void put2(OT* dst, float a, float b);
template <>
__device__ __forceinline__ void put2<_Float16>(_Float16* dst, float a, float b) {
    half2v h;
    h[0] = (_Float16)a;
    h[1] = (_Float16)b;
    *reinterpret_cast<half2v*>(dst) = h;
}
template <>
__device__ __forceinline__ void put2<float>(float* dst, float a, float b) {
    *reinterpret_cast<float2*>(dst) = make_float2(a, b);
}

// Outputs are written once and read by nobody here: non-temporal stores keep
// them from displacing the chunk records in the caches.
__device__ __forceinline__ void store_out(float* p, float x) { __builtin_nontemporal_store(x, p); }
__device__ __forceinline__ void store_out(bf16_t* p, float x) {
    __builtin_nontemporal_store(f32_to_bf16(x).bits, reinterpret_cast<uint16_t*>(p));
}
// fp16 o for the layer epilogue: non-temporal too (plain stores allocate in the
// last-level cache and evict the records the state pass still reads)
__device__ __forceinline__ void store_out(_Float16* p, float x) {
    __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (_Float16)x), reinterpret_cast<uint16_t*>(p));
}

template <typename OT>
struct Frag;
template <>
struct Frag<_Float16> {
    using T = half8;
    __device__ __forceinline__ static T load(const _Float16* p, int g) {
        return *reinterpret_cast<const half8*>(p + 8 * g);
    }
    __device__ __forceinline__ static floatx4 mma(T a, const _Float16* bt, int g, floatx4 acc) {
        half8 b = *reinterpret_cast<const half8*>(bt + 8 * g);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
};
template <>
struct Frag<float> {
    using T = float;
    __device__ __forceinline__ static T load(const float* p, int g) { return p[g]; }
    __device__ __forceinline__ static floatx4 mma(T a, const float* bt, int g, floatx4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, bt[g], acc, 0, 0, 0);
    }
};

// T = (I + A)^-1 for a 64 x 64 strictly lower-triangular A (the UT transform of
// the "Kimi Linear" page, "The constrained DPLR form and the chunkwise
// algorithm"), fp32 in LDS with row pitch AP, by a workgroup of NW >= 4 waves;
// sT and sAt must not overlap.  Only A's strictly lower part is read.  Ends with
// a workgroup barrier; sT's strictly upper blocks hold scratch afterwards.
template <int AP, int NW>
__device__ __forceinline__ void ut_inverse64(float* sT, float* sAt, int wave, int lane) {
    const int gq = lane >> 4, li = lane & 15;
    // Diagonal 16x16 blocks: wave d < 4 inverts I + A for its strictly lower
    // block A as (I - A)(I + A^2)(I + A^4)(I + A^8) (A^16 = 0), four levels of
    // wave-local fp32 tile products.  Its three scratch tiles are off-diagonal
    // blocks of sT that are written only later.  Off-diagonal blocks by 2x2
    // block inversion, first of the two 32x32 halves, then of the whole:
    //   T10 = -T11 A10 T00,  T32 = -T33 A32 T22,
    //   T_hi,lo = -T_hi (A_hi,lo T_lo)   (hi = blocks 2,3; lo = blocks 0,1).
    // Upper blocks of sT serve as scratch and read as zero afterwards.
    {
        auto blk = [&](float* M, int r, int c) { return M + (16 * r) * AP + 16 * c; };
        auto tload = [&](const float* M) {
            floatx4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = M[(4 * gq + r) * AP + li];
            return v;
        };
        auto tstore = [&](float* M, floatx4 v, float sign) {
#pragma unroll
            for (int r = 0; r < 4; ++r) M[(4 * gq + r) * AP + li] = sign * v[r];
        };
        auto prod = [&](floatx4& acc, const float* A, const float* B) {
            mma_tile_f32_rowB(acc, A, AP, B, AP, 16, lane);
        };
        if (wave < 4) {
            const int d = wave;
            // scratch tiles of wave d: (0,1) (0,2) (0,3) | (1,2) (1,3) (2,3) | (2,0) (3,0) (2,1) | (3,1) (3,2) (1,0)
            constexpr int SR[4][3] = {{0, 0, 0}, {1, 1, 2}, {2, 3, 2}, {3, 3, 1}};
            constexpr int SC[4][3] = {{1, 2, 3}, {2, 3, 3}, {0, 0, 1}, {1, 2, 0}};
            float* S0 = blk(sT, SR[d][0], SC[d][0]);
            float* S1 = blk(sT, SR[d][1], SC[d][1]);
            float* S2 = blk(sT, SR[d][2], SC[d][2]);
            const float* Ad = blk(sAt, d, d);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * gq + r;
                const float x = li < row ? Ad[row * AP + li] : 0.f;
                S0[row * AP + li] = x;                          // A
                S1[row * AP + li] = (li == row ? 1.f : 0.f) - x;  // I - A
            }
            wave_lds_sync();
            floatx4 m = zero4();
            prod(m, S0, S0);  // A^2
            tstore(S2, m, 1.f);
            wave_lds_sync();
            m = zero4();
            prod(m, S2, S2);  // A^4
            floatx4 x = tload(S1);
            prod(x, S1, S2);  // (I - A)(I + A^2)
            wave_lds_sync();
            tstore(S0, m, 1.f);
            tstore(S1, x, 1.f);
            wave_lds_sync();
            m = zero4();
            prod(m, S0, S0);  // A^8
            x = tload(S1);
            prod(x, S1, S0);  // ... (I + A^4)
            wave_lds_sync();
            tstore(S2, m, 1.f);
            tstore(S1, x, 1.f);
            wave_lds_sync();
            x = tload(S1);
            prod(x, S1, S2);  // ... (I + A^8)
            tstore(blk(sT, d, d), x, 1.f);
            if (d == 0 || d == 2) {
                // A_{d+1,d} T_dd, kept in S0: (0,1) for d = 0, (2,0) for d = 2
                wave_lds_sync();
                floatx4 y = zero4();
                prod(y, blk(sAt, d + 1, d), blk(sT, d, d));
                tstore(S0, y, 1.f);
            }
        }
        __syncthreads();
        for (int task = wave; task < 6; task += NW) {
            floatx4 acc = zero4();
            switch (task) {
                case 0:  // T10 = -T11 (A10 T00)
                    prod(acc, blk(sT, 1, 1), blk(sT, 0, 1));
                    tstore(blk(sT, 1, 0), acc, -1.f);
                    break;
                case 1:  // T32 = -T33 (A32 T22)
                    prod(acc, blk(sT, 3, 3), blk(sT, 2, 0));
                    tstore(blk(sT, 3, 2), acc, -1.f);
                    break;
                case 2:  // Y21 = A21 T11
                    prod(acc, blk(sAt, 2, 1), blk(sT, 1, 1));
                    tstore(blk(sT, 1, 2), acc, 1.f);
                    break;
                case 3:  // Y31 = A31 T11
                    prod(acc, blk(sAt, 3, 1), blk(sT, 1, 1));
                    tstore(blk(sT, 1, 3), acc, 1.f);
                    break;
                case 4:  // A20 T00 (first term of Y20)
                    prod(acc, blk(sAt, 2, 0), blk(sT, 0, 0));
                    tstore(blk(sT, 0, 2), acc, 1.f);
                    break;
                default:  // A30 T00 (first term of Y30)
                    prod(acc, blk(sAt, 3, 0), blk(sT, 0, 0));
                    tstore(blk(sT, 0, 3), acc, 1.f);
                    break;
            }
        }
        __syncthreads();
        for (int task = wave; task < 4; task += NW) {
            floatx4 acc;
            switch (task) {
                case 0:  // Y20 = A20 T00 + A21 T10
                    acc = tload(blk(sT, 0, 2));
                    prod(acc, blk(sAt, 2, 1), blk(sT, 1, 0));
                    tstore(blk(sT, 0, 2), acc, 1.f);
                    break;
                case 1:  // Y30 = A30 T00 + A31 T10
                    acc = tload(blk(sT, 0, 3));
                    prod(acc, blk(sAt, 3, 1), blk(sT, 1, 0));
                    tstore(blk(sT, 0, 3), acc, 1.f);
                    break;
                case 2:  // T21 = -T22 Y21
                    acc = zero4();
                    prod(acc, blk(sT, 2, 2), blk(sT, 1, 2));
                    tstore(blk(sT, 2, 1), acc, -1.f);
                    break;
                default:  // T31 = -(T32 Y21 + T33 Y31)
                    acc = zero4();
                    prod(acc, blk(sT, 3, 2), blk(sT, 1, 2));
                    prod(acc, blk(sT, 3, 3), blk(sT, 1, 3));
                    tstore(blk(sT, 3, 1), acc, -1.f);
                    break;
            }
        }
        __syncthreads();
        if (wave < 2) {
            floatx4 acc = zero4();
            if (wave == 0) {  // T20 = -T22 Y20
                prod(acc, blk(sT, 2, 2), blk(sT, 0, 2));
                tstore(blk(sT, 2, 0), acc, -1.f);
            } else {  // T30 = -(T32 Y20 + T33 Y30)
                prod(acc, blk(sT, 3, 2), blk(sT, 0, 2));
                prod(acc, blk(sT, 3, 3), blk(sT, 0, 3));
                tstore(blk(sT, 3, 0), acc, -1.f);
            }
        }
        __syncthreads();
    }
}

}  // namespace kda
