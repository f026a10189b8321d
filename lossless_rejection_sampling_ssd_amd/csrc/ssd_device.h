// ssd_device.h -- device helpers for the gfx950 kernels of the SSD / Saguaro round:
// bf16 / fp32 tile loads, order-preserving keys, wave64 reductions (DPP), softmax
// terms with integer offsets, the Philox4x64-10 generator and wave-level radix selects.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr int kWave = 64;        // CDNA wavefront
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kVecPerLane = 8;   // 16-byte vectors each lane keeps in flight per tile
constexpr int kMaxK = 16;
constexpr int kMaxF = 64;

template <int DT> struct ElemTraits;
template <> struct ElemTraits<0> {  // fp32
    static constexpr int kPerVec = 4;
    static constexpr int kBytes = 4;
};
template <> struct ElemTraits<1> {  // bf16
    static constexpr int kPerVec = 8;
    static constexpr int kBytes = 2;
};
template <int DT> constexpr int kTile = kVecPerLane * kWave * ElemTraits<DT>::kPerVec;  // per wave
// Pass 2 (residual sums) works on half tiles: twice the waves for the same bytes, so that
// the arithmetic of early waves overlaps the loads of later ones.
constexpr int kVecPass2 = 4;
template <int DT> constexpr int kTile2 = kVecPass2 * kWave * ElemTraits<DT>::kPerVec;
// A draw picks a block of kDrawBlock consecutive ids first, then the id inside it; a
// pass-2 tile holds whole blocks, a block whole wave vectors (1 bf16, 2 fp32).
constexpr int kDrawBlock = 512;
template <int DT> constexpr int kVecPerBlock = kDrawBlock / (kWave * ElemTraits<DT>::kPerVec);
template <int DT> constexpr int kBlocksPerTile2 = kVecPass2 / kVecPerBlock<DT>;
static_assert(kTile2<0> % kDrawBlock == 0 && kTile2<1> % kDrawBlock == 0, "tiles hold whole draw blocks");

// ---------------------------------------------------------------------------- loads
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// The raw pattern of a vector of -inf elements.
template <int DT>
__device__ __forceinline__ u32x4 neg_inf_vec() {
    const uint32_t w = DT == 1 ? 0xFF80FF80u : 0xFF800000u;
    u32x4 v;
    v.x = v.y = v.z = v.w = w;
    return v;
}

// Raw 16-byte vector of elements [e0, e0 + kPerVec) of a row by element loads, the
// elements at or past V replaced by the -inf pattern.  Every element load reads a
// clamped, in-range id and is unconditional, so all of them are in flight together.
template <int DT>
__device__ __forceinline__ u32x4 load_raw_elems(const char* row, int64_t e0, int V) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    uint32_t w[4];
    if (DT == 1) {
        uint32_t h[N];
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const int64_t id = e0 + e < V ? e0 + e : V - 1;
            h[e] = reinterpret_cast<const uint16_t*>(row)[id];
        }
#pragma unroll
        for (int e = 0; e < N; ++e)
            if (e0 + e >= V) h[e] = 0xFF80u;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = h[2 * q] | (h[2 * q + 1] << 16);
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const int64_t id = e0 + e < V ? e0 + e : V - 1;
            w[e] = reinterpret_cast<const uint32_t*>(row)[id];
        }
#pragma unroll
        for (int e = 0; e < N; ++e)
            if (e0 + e >= V) w[e] = 0xFF800000u;
    }
    u32x4 v;
    v.x = w[0];
    v.y = w[1];
    v.z = w[2];
    v.w = w[3];
    return v;
}
// Bytes [m, m + 16) of the 32 bytes lo ++ hi (little-endian dwords; m in [0, 15]).
__device__ __forceinline__ u32x4 funnel16(u32x4 lo, u32x4 hi, int m) {
    // words wq .. wq + 4 (wq = m / 4) by a two-step rotation, all in registers
    const bool by2 = (m & 8) != 0, by1 = (m & 4) != 0;
    const uint32_t e0 = by2 ? lo.z : lo.x, e1 = by2 ? lo.w : lo.y, e2 = by2 ? hi.x : lo.z;
    const uint32_t e3 = by2 ? hi.y : lo.w, e4 = by2 ? hi.z : hi.x, e5 = by2 ? hi.w : hi.y;
    const uint32_t w[5] = {by1 ? e1 : e0, by1 ? e2 : e1, by1 ? e3 : e2, by1 ? e4 : e3, by1 ? e5 : e4};
    u32x4 r;
    r.x = __builtin_amdgcn_alignbyte(w[1], w[0], (uint32_t)(m & 3));
    r.y = __builtin_amdgcn_alignbyte(w[2], w[1], (uint32_t)(m & 3));
    r.z = __builtin_amdgcn_alignbyte(w[3], w[2], (uint32_t)(m & 3));
    r.w = __builtin_amdgcn_alignbyte(w[4], w[3], (uint32_t)(m & 3));
    return r;
}

template <int DT>
__device__ __forceinline__ void unpack_vec(u32x4 v, float* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if (DT == 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            x[2 * q] = __uint_as_float(w[q] << 16);
            x[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = __uint_as_float(w[q]);
    }
}

// Marks the vectors as rewritten, so that values derived from them before this point
// are recomputed after it instead of being kept in registers.
template <int NV>
__device__ __forceinline__ void opaque_regs(u32x4 (&raw)[NV]) {
#pragma unroll
    for (int j = 0; j < NV; ++j) __asm__ volatile("" : "+v"(raw[j]));
}

// Element e (a compile-time constant after unrolling) of a raw vector, widened to fp32.
template <int DT>
__device__ __forceinline__ float vec_elem(const u32x4& v, int e) {
    if (DT == 1) {
        const uint32_t w = v[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    return __uint_as_float(v[e]);
}
// The NV raw vectors one lane owns in a wave tile starting at element t0
// (vector j covers [t0 + (j*64 + lane)*kPerVec, +kPerVec)), elements at or past V
// replaced by -inf.  VEC: the row is 16-byte aligned.
//  - whole tile in range: unconditional 16-byte loads, issued back to back,
//    non-temporal (each logit is read once per pass);
//  - last tile of an aligned row: vectors wholly in range are loaded as vectors (lanes
//    past the end load the row's first vector instead and discard it, so the loads
//    stay unconditional); the one vector that straddles V, if any, by element loads;
//  - unaligned rows: element loads of clamped ids.
template <int DT, bool VEC, int NV>
__device__ __forceinline__ void load_tile(const char* row, int64_t t0, int V, int lane, u32x4 (&raw)[NV]) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    constexpr int TILE = NV * kWave * N;
    if (VEC && t0 + TILE <= V) {
        const u32x4* base = reinterpret_cast<const u32x4*>(row + t0 * ElemTraits<DT>::kBytes) + lane;
#pragma unroll
        for (int j = 0; j < NV; ++j) raw[j] = __builtin_nontemporal_load(base + j * kWave);
    } else if (VEC) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
            const bool whole = e0 + N <= V;
            const u32x4 v = *reinterpret_cast<const u32x4*>(row + (whole ? e0 : 0) * ElemTraits<DT>::kBytes);
            raw[j] = whole ? v : neg_inf_vec<DT>();
        }
        if (V % N != 0) {
            const int64_t js = ((int64_t)(V / N) * N - t0) / N;  // vector index (j*64 + lane) that straddles V
            if (js >= 0 && js < NV * kWave && js % kWave == lane) {
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    if (j == js / kWave) raw[j] = load_raw_elems<DT>(row, t0 + js * N, V);
            }
        }
    } else {
        // Rows that do not start on a 16-byte boundary.  A vector's bytes start m =
        // row mod 16 bytes into an aligned 16-byte block (the same m for every vector
        // of the row, as vectors are 16 bytes apart), so it is two aligned blocks and a
        // funnel shift by m.  The first load starts at most 15 bytes before the vector,
        // never below the 16-byte-aligned allocation; a tile takes this path only when
        // its last vector's second load ends inside the row's own data (then every
        // vector's does), the row's last tile loads element by element.
        constexpr int ES = ElemTraits<DT>::kBytes;
        const uintptr_t rb = reinterpret_cast<uintptr_t>(row);
        const int m = (int)(rb & 15u);
        const uintptr_t row_end = rb + (uintptr_t)V * ES;
        const int64_t e_last = t0 + (int64_t)(NV * kWave - 1) * N;
        const uintptr_t a_last = (rb + (uintptr_t)(e_last * ES)) & ~(uintptr_t)15;
        if (e_last + N <= V && a_last + 32 <= row_end) {  // uniform over the wave
            // One aligned block per vector; a vector's second block is the first block
            // of the next lane (lane 63: of lane 0 in the next vector, and after the
            // tile's last vector one more block that lane 63 loads itself).
            u32x4 lo[NV];
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
                const uintptr_t a0 = (rb + (uintptr_t)(e0 * ES)) & ~(uintptr_t)15;
                lo[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a0));
            }
            u32x4 tail = lo[NV - 1];
            if (lane == kWave - 1) tail = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a_last + 16));
            const int src = ((lane + 1) & (kWave - 1)) * 4;  // ds_bpermute byte address
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const u32x4 give = (j + 1 < NV && lane == 0) ? lo[j + 1 < NV ? j + 1 : j] : lo[j];
                u32x4 hi;
                hi.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)give.x);
                hi.y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)give.y);
                hi.z = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)give.z);
                hi.w = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)give.w);
                if (j == NV - 1 && lane == kWave - 1) hi = tail;
                raw[j] = funnel16(lo[j], hi, m);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NV; ++j)
                raw[j] = load_raw_elems<DT>(row, t0 + (int64_t)(j * kWave + lane) * N, V);
        }
    }
}

template <int DT>
__device__ __forceinline__ float load_one(const char* row, int64_t id) {
    if (DT == 1) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(row)[id]);
    return reinterpret_cast<const float*>(row)[id];
}

// ---------------------------------------------------------------------------- keys
// Order-preserving map of a float to uint32 (larger float -> larger key), with -0
// mapped like +0 so that equal values compare equal.  Finite and -inf inputs only.
__device__ __forceinline__ uint32_t ord32(float v) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unord32(uint32_t k) {
    uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(b);
}
// 64-bit candidate key: larger value first, then lower id.  Never 0 for a real
// element (ord32(-inf) > 0), so 0 marks an empty slot.
__device__ __forceinline__ uint64_t cand_key(float v, uint32_t id) {
    return ((uint64_t)ord32(v) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu); }
__device__ __forceinline__ float key_val(uint64_t k) { return unord32((uint32_t)(k >> 32)); }

// ---------------------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// A value every lane holds alike, moved to a scalar register so that loops and
// branches on it are scalar (wave-level) control flow, not per-lane masking.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ uint64_t uniform(uint64_t v) {
    return ((uint64_t)uniform((uint32_t)(v >> 32)) << 32) | uniform((uint32_t)v);
}

// ---------------------------------------------------------------------------- wave reductions
// Reductions over the whole wave (all lanes active), result uniform.  Four row shifts
// by 1, 2, 4 and 8 lanes (DPP moves, no LDS round trip) reduce each 16-lane row into
// its last lane; lanes 15, 31, 47 and 63 are then combined as (r0 . r1) . (r2 . r3).
// A shift that would read from outside the row reads the identity instead.  The
// combination order is fixed, so floating-point results are reproducible.
enum { kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118 };

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t ident, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, uint32_t ident, Op op) {
    v = op(v, dpp_u32<kRowShr1>(ident, v));
    v = op(v, dpp_u32<kRowShr2>(ident, v));
    v = op(v, dpp_u32<kRowShr4>(ident, v));
    v = op(v, dpp_u32<kRowShr8>(ident, v));
    return op(op(lane_u32(v, 15), lane_u32(v, 31)), op(lane_u32(v, 47), lane_u32(v, 63)));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce_u32(v, 0u, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ int wave_min_i32(int v) {
    return (int)wave_reduce_u32((uint32_t)v, 0x7FFFFFFFu,
                                [](uint32_t x, uint32_t y) { return (int)x < (int)y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    return wave_reduce_u32(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
    return wave_reduce_u32(v, 0u, [](uint32_t x, uint32_t y) { return x | y; });
}
__device__ __forceinline__ uint32_t wave_and_u32(uint32_t v) {
    return wave_reduce_u32(v, ~0u, [](uint32_t x, uint32_t y) { return x & y; });
}
__device__ __forceinline__ float wave_max_f32(float v) {
    return __uint_as_float(wave_reduce_u32(__float_as_uint(v), 0xFF800000u, [](uint32_t x, uint32_t y) {
        return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
    }));
}
__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
    return ((uint64_t)wave_or_u32((uint32_t)(v >> 32)) << 32) | wave_or_u32((uint32_t)v);
}
__device__ __forceinline__ uint64_t wave_and64(uint64_t v) {
    return ((uint64_t)wave_and_u32((uint32_t)(v >> 32)) << 32) | wave_and_u32((uint32_t)v);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64_zero(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = dpp_u32<CTRL>(0u, (uint32_t)b), hi = dpp_u32<CTRL>(0u, (uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double lane_f64(double v, int l) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    return __longlong_as_double((long long)(((uint64_t)lane_u32((uint32_t)(b >> 32), l) << 32) |
                                            lane_u32((uint32_t)b, l)));
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
    return ((uint64_t)lane_u32((uint32_t)(v >> 32), l) << 32) | lane_u32((uint32_t)v, l);
}
// Sum over the wave in fp64 (fixed order).
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64_zero<kRowShr1>(v);
    v += dpp_f64_zero<kRowShr2>(v);
    v += dpp_f64_zero<kRowShr4>(v);
    v += dpp_f64_zero<kRowShr8>(v);
    return (lane_f64(v, 15) + lane_f64(v, 31)) + (lane_f64(v, 47) + lane_f64(v, 63));
}
// Inclusive prefix sums over lanes in lane order (all lanes active): row shifts give
// the prefix within each 16-lane row, then the totals of the rows below are added.
__device__ __forceinline__ uint32_t wave_prefix_u32(uint32_t v) {
    v += dpp_u32<kRowShr1>(0u, v);
    v += dpp_u32<kRowShr2>(0u, v);
    v += dpp_u32<kRowShr4>(0u, v);
    v += dpp_u32<kRowShr8>(0u, v);
    const uint32_t r0 = lane_u32(v, 15), r1 = lane_u32(v, 31), r2 = lane_u32(v, 47);
    const int row = lane_id() >> 4;
    return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}
__device__ __forceinline__ double wave_prefix_f64(double v) {
    v += dpp_f64_zero<kRowShr1>(v);
    v += dpp_f64_zero<kRowShr2>(v);
    v += dpp_f64_zero<kRowShr4>(v);
    v += dpp_f64_zero<kRowShr8>(v);
    const double r0 = lane_f64(v, 15), r1 = lane_f64(v, 31), r2 = lane_f64(v, 47);
    const int row = lane_id() >> 4;
    const double below = row == 0 ? 0.0 : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
    return v + below;
}

__device__ __forceinline__ int wave_popc(bool p) { return __popcll(__ballot(p)); }
// Number of lanes below this one with p set.
__device__ __forceinline__ int lanes_below(bool p) {
    const uint64_t m = __ballot(p);
    return __popcll(m & ((1ull << lane_id()) - 1ull));
}

// ---------------------------------------------------------------------------- softmax terms
// With c = log2(e)/T every term of a row is 2^{z c - o} for an integer-valued offset
// o = rint(m c) taken from a maximum m, so the exponent is formed by one fma with a
// single rounding and partial sums under different offsets merge exactly by
// ldexp.  o(-inf) = 0 (such a partial has no mass).
__device__ __forceinline__ float offset_of(float m, float c) { return m == -INFINITY ? 0.f : rintf(m * c); }
// max(a, b, c) for non-NaN operands, as one v_maximum3_f32 (no canonicalisation).
__device__ __forceinline__ float fmax3_nan(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float term(float z, float c, float o) { return __builtin_amdgcn_exp2f(fmaf(z, c, -o)); }

// Sum of 2^{z c - o(M)} for the union of two partials (m1, s1), (m2, s2) whose sums are
// relative to o(m1), o(m2).
__device__ __forceinline__ void merge_partial(float& m, double& s, float m2, double s2, float c) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) {
        m = M;
        s = 0.0;
        return;
    }
    const float oM = offset_of(M, c);
    const double a = (m == -INFINITY) ? 0.0 : ldexp(s, (int)(offset_of(m, c) - oM));
    const double b = (m2 == -INFINITY) ? 0.0 : ldexp(s2, (int)(offset_of(m2, c) - oM));
    s = a + b;
    m = M;
}

// ---------------------------------------------------------------------------- Philox
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round two 64x64->128
// products with the published multipliers, key bumped by the published Weyl
// constants; returns the first output word of counter (round, b, i, w3) under key
// (seed, purpose).
__device__ __forceinline__ uint64_t philox_word0(uint64_t seed, uint64_t round, uint32_t purpose,
                                                 uint64_t b, uint64_t i, uint64_t w3 = 0) {
    uint64_t c0 = round, c1 = b, c2 = i, c3 = w3;
    uint64_t k0 = seed, k1 = purpose;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t lo0 = 0xD2E7470EE14C6C93ull * c0;
        const uint64_t hi0 = __umul64hi(0xD2E7470EE14C6C93ull, c0);
        const uint64_t lo1 = 0xCA5A826395121157ull * c2;
        const uint64_t hi1 = __umul64hi(0xCA5A826395121157ull, c2);
        const uint64_t n0 = hi1 ^ c1 ^ k0;
        const uint64_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B97F4A7C15ull;
        k1 += 0xBB67AE8584CAA73Bull;
    }
    return c0;
}
// u in [0, 1) with 24 random bits, exact in fp32.  w3 = 0: the uniform of a test or
// of a draw's block; w3 = 1: a draw's second uniform (the id inside the block).
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t round, uint32_t purpose, uint64_t b,
                                                uint64_t i, uint64_t w3 = 0) {
    return (float)(uint32_t)(philox_word0(seed, round, purpose, b, i, w3) >> 40) * (1.0f / 16777216.0f);
}
__device__ __forceinline__ uint32_t philox_u32(uint64_t seed, uint64_t round, uint32_t purpose, uint64_t b,
                                               uint64_t i) {
    return (uint32_t)(philox_word0(seed, round, purpose, b, i) >> 32);
}

// ---------------------------------------------------------------------------- select
// The F-th largest of the distinct nonzero 64-bit keys held by a whole wave in
// KREG register slots per lane (0 = empty slot), by a most-significant-bit-first
// radix select that only tests bits where the keys differ.  Returns 0 when there
// are at most F keys (every key is in).
template <int KREG>
__device__ inline uint64_t wave_select_regs(const uint64_t (&k)[KREG], int F) {
    int n = 0;
    uint64_t orv = 0ull, andv = ~0ull;
#pragma unroll
    for (int s = 0; s < KREG; ++s) {
        n += wave_popc(k[s] != 0ull);
        if (k[s] != 0ull) {
            orv |= k[s];
            andv &= k[s];
        }
    }
    if (n <= F) return 0ull;
    orv = wave_or64(orv);
    andv = wave_and64(andv);
    uint64_t diff = orv ^ andv;
    uint64_t T = andv & ~diff;
    while (diff) {
        const int bit = 63 - __clzll(diff);
        diff &= ~(1ull << bit);
        const uint64_t cand = T | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int s = 0; s < KREG; ++s) cnt += wave_popc(k[s] >= cand);
        if (cnt >= F) T = cand;
    }
    return T;
}

// Same for one nonzero 32-bit key per lane (0 = no key).
// With max_bits below 32 only the max_bits highest bits in which the keys differ are
// resolved and the rest are left 0: a lower bound of the F-th largest key that still
// has at least F keys at or above it.
// The F-th largest of the nonzero keys the wave holds in R registers per lane (0 when at
// most F are nonzero), by the same most-significant-bit-first search over the bits
// where the keys differ.  Only the differing bits in bit_mask are resolved; the others
// are left at the bits every key shares, which gives a lower bound of the F-th largest
// key with at least F keys at or above it.
template <int R>
__device__ inline uint32_t wave_select_regs_u32(const uint32_t (&k)[R], int F, uint32_t bit_mask = ~0u) {
    int n = 0;
    uint32_t orv = 0u, andv = ~0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        n += wave_popc(k[r] != 0u);
        orv |= k[r];
        andv &= k[r] ? k[r] : ~0u;
    }
    if (n <= F) return 0u;
    orv = wave_or_u32(orv);
    andv = wave_and_u32(andv);
    uint32_t diff = orv ^ andv;
    uint32_t T = andv & ~diff;
    diff &= bit_mask;
    for (int it = 0; diff && it < 32; ++it) {
        const int bit = 31 - __clz(diff);
        diff &= ~(1u << bit);
        const uint32_t cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) cnt += wave_popc(k[r] >= cand);
        if (cnt >= F) T = cand;
    }
    return T;
}

__device__ inline uint32_t wave_select_u32(uint32_t k, int F, int max_bits = 32) {
    const int n = wave_popc(k != 0u);
    if (n <= F) return 0u;
    uint32_t orv = k, andv = k ? k : ~0u;
    orv = wave_or_u32(orv);
    andv = wave_and_u32(andv);
    uint32_t diff = orv ^ andv;
    uint32_t T = andv & ~diff;
    for (int it = 0; diff && it < max_bits; ++it) {
        const int bit = 31 - __clz(diff);
        diff &= ~(1u << bit);
        const uint32_t cand = T | (1u << bit);
        if (wave_popc(k >= cand) >= F) T = cand;
    }
    return T;
}

}  // namespace ssd
