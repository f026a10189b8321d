// ssd_kernels.hip -- gfx950 kernels of the verify-and-pre-speculate round of
// Speculative Speculative Decoding with the Saguaro algorithm.
//
// Data flow of one round (two streaming kernels):
//  pass 1  every row of the target and draft logits [B, K+1, V] is read once.  Each
//          256-thread block (4 wave64s) owns one vocabulary chunk of one row; each
//          lane keeps 8 x 16-byte vectors in registers.  Per chunk it computes the
//          softmax partial (max, sum of 2^{z c - o}), the lowest-id argmax, and for
//          draft rows the chunk's exact top-F keys (wave radix select on lane maxima,
//          LDS candidate staging, wave radix select of the top F).  The last block of
//          a sequence (completion counter) merges its rows: softmax statistics, cache
//          ids S_k (sorted, ties to the lower id), M_k, the Saguaro normaliser Z_k and
//          the lossless verification of the K draft tokens.
//  pass 2  only the rows the bonus needs (target row k, plus draft row k when k < K)
//          are read again.  Each block sums the residual max(p - q', 0) per wave
//          segment of its chunk; the last block of the sequence locates the segment
//          where the running sum crosses u * sum, rescans that segment to find the
//          bonus id, and performs the cache lookup.
// Normalisers, cached masses, Z and every running sum that decides an integer are
// kept in fp64; per-element terms are fp32 exp2 of an exactly formed exponent.
// The separate C-ABI calls reuse the same device code, so their results are
// bit-identical to the fused round.
#include "ssd_device.h"
#include "ssd_kernels.h"

#include <climits>

namespace ssd {

enum { kPurposeAccept = 0, kPurposeBonus = 1, kPurposeDraft = 2, kPurposeFallback = 3 };
enum { kErrTokenRange = 1, kErrQprimeZero = 2, kErrLenRange = 4 };

int chunk_elems(int dtype) { return dtype == 1 ? kChunk<1> : kChunk<0>; }
int blocks_per_row(int dtype, int V) {
    const int c = chunk_elems(dtype);
    return (V + c - 1) / c;
}

// ============================================================================ shared pieces
// Row normalisation from the exchanged statistics (row max m, row sum
// s = sum_x 2^{(z_x - m) c}): p(x) = term(z_x, c, o) * inv with o = rint(m c).
// Sums relative to o(m) and the standard row sum differ by the factor
// f = 2^{o - m c} (|o - m c| <= 1/2); both directions use the same fp32 factor, so
// a sum converted to the standard form and back changes only by fp64 rounding.
__device__ __forceinline__ double offset_factor(float m, float c, float o) {
    return (double)__builtin_amdgcn_exp2f((float)((double)o - (double)m * (double)c));
}
struct RowNorm {
    float o;
    double inv;
};
__device__ __forceinline__ RowNorm row_norm(float m, double s_std, float c) {
    RowNorm r;
    r.o = offset_of(m, c);
    r.inv = offset_factor(m, c, r.o) / s_std;
    return r;
}
// Standard row sum from a sum relative to o(m).
__device__ __forceinline__ double std_sum(float m, double s_rel, float c) {
    return s_rel * offset_factor(m, c, offset_of(m, c));
}

__device__ __forceinline__ void publish_partial(RowPartial* p, float m, int arg, double s) {
    const uint64_t w = (uint64_t)__float_as_uint(m) | ((uint64_t)(uint32_t)arg << 32);
    publish(reinterpret_cast<uint64_t*>(p), w);
    publish(&p->s, s);
}
__device__ __forceinline__ RowPartial observe_partial(const RowPartial* p) {
    const uint64_t w = observe(reinterpret_cast<const uint64_t*>(p));
    RowPartial r;
    r.m = __uint_as_float((uint32_t)w);
    r.arg = (int)(uint32_t)(w >> 32);
    r.s = observe(&p->s);
    return r;
}

// Softmax statistics of a row from its per-chunk partials, merged in chunk order.
// Returns the sum relative to o(m).
__device__ inline void combine_partials(const RowPartial* P, int nb, float c, float& m, double& s, int& arg) {
    RowPartial q = observe_partial(P);
    m = q.m;
    s = q.s;
    arg = q.arg;
    for (int j = 1; j < nb; ++j) {
        q = observe_partial(P + j);
        if (q.m > m || (q.m == m && q.arg < arg)) arg = q.arg;
        merge_partial(m, s, q.m, q.s, c);
    }
}

// Cache lookup of one verified outcome (k, tok) by one wave, plus the uniform
// fallback draft on a miss.
__device__ inline void lookup_wave(int b, int K, int V, int k, int tok, const int* F, const int* O, int Bf,
                                   const int32_t* cache_ids, int fallback, uint64_t seed, uint64_t round,
                                   uint8_t* hit, int32_t* slot, int32_t* fb) {
    const int lane = lane_id();
    bool match = false;
    int Ok = 0;
    if (k >= 0 && k <= K) {
        Ok = O[k];
        if (lane < F[k]) match = cache_ids[(int64_t)b * Bf + Ok + lane] == tok;
    }
    const uint64_t mk = __ballot(match);
    const bool h = mk != 0ull;
    if (lane == 0) {
        hit[b] = h ? 1 : 0;
        slot[b] = h ? Ok + (__ffsll((long long)mk) - 1) : -1;
    }
    for (int j = lane; j < K; j += kWave) {
        int32_t t = -1;
        if (!h && fallback) {
            const uint64_t u32 = philox_u32(seed, round, kPurposeFallback, (uint64_t)b, (uint64_t)j);
            t = (int32_t)((u32 * (uint64_t)V) >> 32);
        }
        fb[(int64_t)b * K + j] = t;
    }
}

// Verification of the K draft tokens of sequence b by one wave: lane i < K tests
// position i with that position's row statistics.  Returns the accepted length k
// (same in every lane); writes accept_prob and the OR of the error bits to *errs.
template <int DT>
__device__ inline int verify_wave(int b, int K, int V, const char* p_row_i, const char* q_row_i, int d, float mp,
                                  double sp, int argp, float mq, double sq, double Zi, bool in_cache, float C, float c,
                                  int greedy, uint64_t seed, uint64_t round, float* accept_prob, int* errs) {
    const int i = lane_id();
    const bool act = i < K;
    int err = 0;
    bool ok = act;
    double ratio = 0.0;
    if (act && (d < 0 || d >= V)) {
        err |= kErrTokenRange;
        ok = false;
    }
    if (ok) {
        if (greedy) {
            ratio = (d == argp) ? 1.0 : 0.0;
        } else {
            const RowNorm np = row_norm(mp, sp, c), nq = row_norm(mq, sq, c);
            const double p = (double)term(load_one<DT>(p_row_i, d), c, np.o) * np.inv;
            const double q = (double)term(load_one<DT>(q_row_i, d), c, nq.o) * nq.inv;
            const double qp = q * (in_cache ? (double)C : 1.0) / Zi;
            if (!(qp > 0.0)) {
                err |= kErrQprimeZero;
                ok = false;
            } else {
                ratio = p / qp;
            }
        }
    }
    bool acc = false;
    if (ok) {
        if (greedy)
            acc = ratio == 1.0;
        else
            acc = (double)philox_uniform(seed, round, kPurposeAccept, (uint64_t)b, (uint64_t)i) < ratio;
    }
    const uint64_t rej = __ballot(act && !acc);
    const int k = rej ? (__ffsll((long long)rej) - 1) : K;
    if (act && accept_prob) accept_prob[(int64_t)b * K + i] = (float)(ratio < 1.0 ? ratio : 1.0);
    int e = err;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) e |= __shfl_xor(e, m, kWave);
    *errs = e;
    return k;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Merges nb per-chunk lists of F keys (Fmax slots each, 0 = empty) into the row's
// top F, returned sorted: lane j holds the j-th largest key (0 past the end).
// xchg: 64 uint64 of LDS private to the calling wave.
__device__ inline uint64_t merge_topf(const uint64_t* lists, int nb, int Fmax, int F, uint64_t* xchg) {
    const int lane = lane_id();
    constexpr int KR = 4;
    uint64_t keep = 0ull;
    const int per_batch = ((KR - 1) * kWave) / F;
    for (int l0 = 0; l0 < nb; l0 += per_batch) {
        const int l1 = min(nb, l0 + per_batch);
        const int n = (l1 - l0) * F;
        uint64_t k[KR];
        k[0] = keep;
#pragma unroll
        for (int s = 1; s < KR; ++s) {
            const int idx = (s - 1) * kWave + lane;
            k[s] = idx < n ? observe(lists + (int64_t)(l0 + idx / F) * Fmax + idx % F) : 0ull;
        }
        const uint64_t T = wave_select_regs<KR>(k, F);
        int written = 0;
#pragma unroll
        for (int s = 0; s < KR; ++s) {
            const bool take = k[s] != 0ull && k[s] >= T;
            const int pos = written + lanes_below(take);
            if (take && pos < kWave) xchg[pos] = k[s];
            written += wave_popc(take);
        }
        wave_sync_lds();
        keep = lane < min(written, F) ? xchg[lane] : 0ull;
        wave_sync_lds();
    }
    return wave_sort_desc(keep);
}

// Cache keys, cached mass M = sum q(x) over them of one draft row, by one wave.
// Writes the sorted ids to ids_out[0..F) (and ids_lds if given).
__device__ inline double cache_row(const uint64_t* lists, int nb, int Fmax, int F, float mq, double sq, float c,
                                   int greedy, int32_t* ids_out, int* ids_lds, uint64_t* xchg) {
    const int lane = lane_id();
    if (F <= 0) return 0.0;
    const uint64_t key = merge_topf(lists, nb, Fmax, F, xchg);
    const int id = key ? (int)key_id(key) : -1;
    if (lane < F) {
        ids_out[lane] = id;
        if (ids_lds) ids_lds[lane] = id;
    }
    double t = 0.0;
    if (lane < F && key) {
        if (greedy) {
            t = lane == 0 ? 1.0 : 0.0;
        } else {
            const RowNorm nq = row_norm(mq, sq, c);
            t = (double)term(key_val(key), c, nq.o) * nq.inv;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) t += __shfl_xor(t, m, kWave);
    return t;
}

// ============================================================================ pass 1
struct FinShared {
    float m[2][kMaxK + 1];
    double s[2][kMaxK + 1];
    int arg[2][kMaxK + 1];
    double Z[kMaxK + 1];
    int ids[kMaxK + 1][kMaxF];
    uint64_t xchg[kWavesPerBlock][kWave];
};

template <int DT>
__device__ void finalize_sequence(const Pass1Args& a, int b, FinShared& fs) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int K1 = a.K1, K = K1 - 1;
    const SeqFinal& f = a.fin;
    const RowPartial* part = a.part + (int64_t)b * a.part_stride;
    const uint64_t* topk = a.topk + (int64_t)b * a.topk_stride;

    // row statistics of both models
    if (tid < 2 * K1) {
        const int model = tid / K1, i = tid % K1;
        const int64_t r = (int64_t)b * K1 + i;
        float m;
        double s;
        int arg;
        combine_partials(part + (int64_t)(model * K1 + i) * a.nb, a.nb, a.c, m, s, arg);
        s = a.greedy ? 1.0 : std_sum(m, s, a.c);
        fs.m[model][i] = m;
        fs.s[model][i] = s;
        fs.arg[model][i] = arg;
        if (model) {
            f.q_max[r] = m;
            f.q_sum[r] = s;
            if (f.q_arg) f.q_arg[r] = arg;
        } else {
            f.p_max[r] = m;
            f.p_sum[r] = s;
            if (f.p_arg) f.p_arg[r] = arg;
        }
    }
    __syncthreads();

    // speculation cache per acceptance length, cached mass and Saguaro normaliser
    for (int i = wave; i < K1; i += kWavesPerBlock) {
        const int64_t r = (int64_t)b * K1 + i;
        const double M = cache_row(topk + (int64_t)i * a.nb * a.Fmax, a.nb, a.Fmax, a.F[i], fs.m[1][i], fs.s[1][i],
                                   a.c, a.greedy, f.cache_ids + (int64_t)b * f.Bf + a.O[i], fs.ids[i], fs.xchg[wave]);
        const double Z = 1.0 - (1.0 - (double)f.C) * M;
        if (lane == 0) {
            f.cache_mass[r] = M;
            f.Z[r] = Z;
            fs.Z[i] = Z;
        }
    }
    __syncthreads();

    if (wave != 0) return;
    const int i = lane;
    const bool act = i < K;
    const int ic = act ? i : 0;
    const int64_t ri = (int64_t)b * K1 + ic;
    const int d = act ? f.draft[(int64_t)b * K + i] : 0;
    bool in_cache = false;
    for (int j = 0; j < a.F[ic]; ++j) in_cache |= fs.ids[ic][j] == d;
    int errs;
    const int k = verify_wave<DT>(b, K, a.V, a.logits[0] + ri * a.ld_bytes, a.logits[1] + ri * a.ld_bytes, d,
                                  fs.m[0][ic], fs.s[0][ic], fs.arg[0][ic], fs.m[1][ic], fs.s[1][ic], fs.Z[ic],
                                  in_cache, f.C, a.c, a.greedy, f.seed, f.round, f.accept_prob, &errs);
    if (lane == 0) {
        f.accept_len[b] = k;
        if (f.dev_err && errs) f.dev_err[b] |= errs;
    }
    if (a.greedy) {
        const int tok = fs.arg[0][k];
        if (lane == 0) {
            f.bonus[b] = tok;
            if (f.resid_mass) f.resid_mass[b] = 1.0;
        }
        lookup_wave(b, K, a.V, k, tok, a.F, a.O, f.Bf, f.cache_ids, f.fallback, f.seed, f.round, f.hit, f.slot,
                    f.fallback_tokens);
    }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void pass1_kernel(const Pass1Args a) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    __shared__ float sh_m[kWavesPerBlock];
    __shared__ double sh_s[kWavesPerBlock];
    __shared__ int sh_a[kWavesPerBlock];
    __shared__ uint64_t sh_best[kWavesPerBlock];
    __shared__ uint64_t sh_cand[kWavesPerBlock * kCandCap];
    __shared__ int sh_ncand;
    __shared__ int sh_overflow;
    __shared__ int sh_last;
    __shared__ FinShared fs;

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    int bid = blockIdx.x;
    const int blk = bid % a.nb;
    bid /= a.nb;
    const int i = bid % a.K1;
    bid /= a.K1;
    const int model = bid % a.nmodel;
    const int b = bid / a.nmodel;
    const int64_t r = (int64_t)b * a.K1 + i;
    const char* row = a.logits[model] + r * a.ld_bytes;
    const int64_t tile0 = (int64_t)blk * kChunk<DT> + (int64_t)wave * kTile<DT>;
    const int V = a.V;
    const float c = a.c;

    if (tid == 0) {
        sh_ncand = 0;
        sh_overflow = 0;
    }

    float x[kVecPerLane][N];
    {
        u32x4 raw[kVecPerLane];
        load_tile<DT, VEC>(row, tile0, V, lane, raw);
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) unpack_vec<DT>(raw[j], x[j]);
    }

    float m_lane = -INFINITY;
#pragma unroll
    for (int j = 0; j < kVecPerLane; ++j)
#pragma unroll
        for (int e = 0; e < N; ++e) m_lane = fmaxf(m_lane, x[j][e]);

    int arg = INT_MAX;
    if (a.want_arg) {
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j)
#pragma unroll
            for (int e = 0; e < N; ++e) {
                const int64_t id = tile0 + (int64_t)(j * kWave + lane) * N + e;
                if (arg == INT_MAX && id < V && x[j][e] == m_lane) arg = (int)id;
            }
    }

    double s = 0.0;
    if (!a.greedy && m_lane != -INFINITY) {
        const float o = offset_of(m_lane, c);
        float vs[kVecPerLane];
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) {
            float t[N];
#pragma unroll
            for (int e = 0; e < N; ++e) t[e] = term(x[j][e], c, o);
#pragma unroll
            for (int w = N / 2; w >= 1; w >>= 1)
#pragma unroll
                for (int e = 0; e < w; ++e) t[e] += t[e + w];
            vs[j] = t[0];
        }
#pragma unroll
        for (int w = kVecPerLane / 2; w >= 1; w >>= 1)
#pragma unroll
            for (int j = 0; j < w; ++j) vs[j] += vs[j + w];
        s = (double)vs[0];
    }

    // ---- top-F candidates of this wave's tile (draft rows of the cache): the F-th
    // largest lane maximum bounds the tile's top F from below.
    const int F = a.F[i];
    const bool do_topf = (model == a.topf_model) && F > 0;
    if (do_topf) {
        const bool lane_valid = tile0 + (int64_t)lane * N < V;
        const uint32_t tau = wave_select_u32(lane_valid ? ord32(m_lane) : 0u, F);
        const float tauf = tau ? unord32(tau) : -INFINITY;
        const int id0 = (int)tile0 + lane * N;
        uint32_t mask[kVecPerLane];
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) {
            uint32_t mk = 0u;
#pragma unroll
            for (int e = 0; e < N; ++e) mk |= (x[j][e] >= tauf && id0 + j * kWave * N + e < V) ? (1u << e) : 0u;
            mask[j] = mk;
            cnt += __popc(mk);
        }
        int incl = cnt;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        const int tot = __shfl(incl, kWave - 1, kWave);
        int base = 0;
        if (lane == 0) base = atomicAdd(&sh_ncand, tot);
        base = __shfl(base, 0, kWave);
        if (base + tot > kWavesPerBlock * kCandCap) {
            if (lane == 0) sh_overflow = 1;
        } else if (cnt) {
            int pos = base + incl - cnt;
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                uint32_t mk = mask[j];
                while (mk) {
                    const int e = __ffs(mk) - 1;
                    mk &= mk - 1u;
                    float v = x[j][0];
#pragma unroll
                    for (int q = 1; q < N; ++q) v = (e == q) ? x[j][q] : v;
                    sh_cand[pos++] = cand_key(v, (uint32_t)(id0 + j * kWave * N + e));
                }
            }
        }
    }

    // ---- wave partial
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m_lane, off, kWave);
        const double s2 = __shfl_xor(s, off, kWave);
        const int a2 = __shfl_xor(arg, off, kWave);
        if (m2 > m_lane || (m2 == m_lane && a2 < arg)) arg = a2;
        merge_partial(m_lane, s, m2, s2, c);
    }
    if (lane == 0) {
        sh_m[wave] = m_lane;
        sh_s[wave] = s;
        sh_a[wave] = arg;
    }
    __syncthreads();

    uint64_t* out_list = a.topk + (int64_t)b * a.topk_stride + ((int64_t)i * a.nb + blk) * a.Fmax;
    if (do_topf) {
        if (!sh_overflow) {
            if (wave == 0) {
                const int n = sh_ncand;
                const uint64_t T = wave_select_lds(sh_cand, n, F);
                int written = 0;
                for (int j0 = 0; j0 < n; j0 += kWave) {
                    const int j = j0 + lane;
                    const uint64_t kk = j < n ? sh_cand[j] : 0ull;
                    const bool take = kk != 0ull && kk >= T;
                    const int pos = written + lanes_below(take);
                    if (take && pos < F) publish(out_list + pos, kk);
                    written += wave_popc(take);
                }
                for (int j = written + lane; j < F; j += kWave) publish(out_list + j, (uint64_t)0);
            }
        } else {
            // Too many tied candidates for LDS (e.g. near-constant logits): exact
            // selection by F rounds of a block-wide maximum below the previous key,
            // re-reading the chunk.
            uint64_t prev = ~0ull;
#pragma unroll 1
            for (int t = 0; t < F; ++t) {
                uint64_t best = 0ull;
#pragma unroll 1
                for (int j = 0; j < kVecPerLane; ++j) {
                    const int64_t e0 = tile0 + (int64_t)(j * kWave + lane) * N;
#pragma unroll 1
                    for (int e = 0; e < N; ++e) {
                        if (e0 + e < V) {
                            const uint64_t kk = cand_key(load_one<DT>(row, e0 + e), (uint32_t)(e0 + e));
                            if (kk < prev && kk > best) best = kk;
                        }
                    }
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    const uint64_t o = __shfl_xor(best, off, kWave);
                    best = o > best ? o : best;
                }
                if (lane == 0) sh_best[wave] = best;
                __syncthreads();
                best = sh_best[0];
#pragma unroll
                for (int w = 1; w < kWavesPerBlock; ++w) best = sh_best[w] > best ? sh_best[w] : best;
                __syncthreads();
                if (tid == 0) publish(out_list + t, best);
                prev = best;
            }
        }
    }

    // ---- block partial
    if (tid == 0) {
        float bm = sh_m[0];
        double bs = sh_s[0];
        int ba = sh_a[0];
#pragma unroll
        for (int w = 1; w < kWavesPerBlock; ++w) {
            if (sh_m[w] > bm || (sh_m[w] == bm && sh_a[w] < ba)) ba = sh_a[w];
            merge_partial(bm, bs, sh_m[w], sh_s[w], c);
        }
        publish_partial(a.part + (int64_t)b * a.part_stride + (int64_t)(model * a.K1 + i) * a.nb + blk, bm, ba, bs);
    }
    if (!a.seq_counter) return;

    // ---- fused round: the last block of sequence b finishes the sequence
    wait_stores();
    __syncthreads();
    if (tid == 0) {
        const unsigned total = (unsigned)(a.nmodel * a.K1 * a.nb);
        const unsigned old = arrive(&a.seq_counter[b]);
        sh_last = (old == total - 1u);
        if (sh_last) publish(&a.seq_counter[b], 0u);
    }
    __syncthreads();
    if (!sh_last) return;
    finalize_sequence<DT>(a, b, fs);
}

// ============================================================================ pass 2
enum { kWResid = 0, kWP = 1, kWQprime = 2 };

struct WParams {
    float c;
    float op, oq;       // offsets of the target / draft rows
    double inv_p;       // p(x) = term(z_p, c, op) * inv_p
    double sc_q, sc_qC; // q'(x) = term(z_q, c, oq) * (sc_qC if cached else sc_q)
};

__device__ inline WParams make_wparams(const Pass2Args& a, int64_t r) {
    WParams w;
    w.c = a.c;
    if (a.mode == 0) {
        const RowNorm np = row_norm(a.p_max[r], a.p_sum[r], a.c);
        w.op = np.o;
        w.inv_p = np.inv;
    } else {
        w.op = 0.f;
        w.inv_p = 0.0;
    }
    const RowNorm nq = row_norm(a.q_max[r], a.q_sum[r], a.c);
    w.oq = nq.o;
    w.sc_q = nq.inv / a.Z[r];
    w.sc_qC = w.sc_q * (double)a.C;
    return w;
}

// Weight of one element for the inverse-CDF scan (fp64); *pw receives p(x).
template <int MODE>
__device__ __forceinline__ double elem_weight_t(const WParams& w, float zp, float zq, bool in_cache, double* pw) {
    double p = 0.0;
    if (MODE != kWQprime) p = (double)term(zp, w.c, w.op) * w.inv_p;
    *pw = p;
    if (MODE == kWP) return p;
    const double q = (double)term(zq, w.c, w.oq) * (in_cache ? w.sc_qC : w.sc_q);
    if (MODE == kWQprime) return q;
    const double d = p - q;
    return d > 0.0 ? d : 0.0;
}
__device__ __forceinline__ double elem_weight(int mode, const WParams& w, float zp, float zq, bool in_cache,
                                              double* pw) {
    if (mode == kWResid) return elem_weight_t<kWResid>(w, zp, zq, in_cache, pw);
    if (mode == kWP) return elem_weight_t<kWP>(w, zp, zq, in_cache, pw);
    return elem_weight_t<kWQprime>(w, zp, zq, in_cache, pw);
}

// Membership bitmap (LDS, kChunk/32 words) of the cached ids of a row that fall in
// [c0, c0 + chunk).
template <int DT>
__device__ inline void clear_bitmap(uint32_t* bits, int t, int nthreads) {
    for (int w = t; w < kChunk<DT> / 32; w += nthreads) bits[w] = 0u;
}
template <int DT>
__device__ inline void set_bitmap(uint32_t* bits, int64_t c0, const int32_t* ids, int F, int t, int nthreads) {
    for (int j = t; j < F; j += nthreads) {
        const int64_t id = ids[j];
        if (id >= c0 && id < c0 + kChunk<DT>) atomicOr(&bits[(id - c0) >> 5], 1u << ((id - c0) & 31));
    }
}

// Weights of one lane's vector (N elements starting at e0) of a tile, from the
// raw vectors of the target (rp) and draft (rq) rows.
template <int DT>
__device__ __forceinline__ void vec_weights(int mode, const WParams& wp, u32x4 rp, u32x4 rq, int64_t e0, int V,
                                            const uint32_t* bits, int64_t c0, double* w, double* p) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    float zp[N], zq[N];
    unpack_vec<DT>(rp, zp);
    unpack_vec<DT>(rq, zq);
    uint32_t cbits = 0u;
    if (mode != kWP) cbits = bits[(e0 - c0) >> 5] >> ((e0 - c0) & 31);
#pragma unroll
    for (int e = 0; e < N; ++e) {
        w[e] = elem_weight(mode, wp, zp[e], zq[e], (cbits >> e) & 1u, &p[e]);
        if (e0 + e >= V) {
            w[e] = 0.0;
            p[e] = 0.0;
        }
    }
}

template <int DT, bool VEC>
__device__ __forceinline__ void load_pair(int mode, const char* prow, const char* qrow, int64_t e0, int V, u32x4& rp,
                                          u32x4& rq) {
    const u32x4 ninf = {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
    rp = mode != kWQprime ? load_raw<DT, VEC>(prow, e0, V) : ninf;
    rq = mode != kWP ? load_raw<DT, VEC>(qrow, e0, V) : ninf;
}

// Sums over one lane's part of a wave tile: sw of the weights, sp of p(x).
template <int DT, bool VEC, int MODE>
__device__ __forceinline__ void tile_sums(const WParams& wp, const char* prow, const char* qrow, int64_t tile0, int V,
                                          const uint32_t* bits, int64_t c0, double& sw, double& sp) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int lane = lane_id();
    u32x4 rp[kVecPerLane], rq[kVecPerLane];
    if (MODE != kWQprime) load_tile<DT, VEC>(prow, tile0, V, lane, rp);
    if (MODE != kWP) load_tile<DT, VEC>(qrow, tile0, V, lane, rq);
#pragma unroll
    for (int j = 0; j < kVecPerLane; ++j) {
        const int64_t e0 = tile0 + (int64_t)(j * kWave + lane) * N;
        float zp[N], zq[N];
        if (MODE != kWQprime) unpack_vec<DT>(rp[j], zp);
        if (MODE != kWP) unpack_vec<DT>(rq[j], zq);
        uint32_t cbits = 0u;
        if (MODE != kWP) cbits = bits[(e0 - c0) >> 5] >> ((e0 - c0) & 31);
        double vw = 0.0, vp = 0.0;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            double p;
            const double w = elem_weight_t<MODE>(wp, MODE != kWQprime ? zp[e] : 0.f, MODE != kWP ? zq[e] : 0.f,
                                                 (cbits >> e) & 1u, &p);
            if (e0 + e < V) {
                vw += w;
                vp += p;
            }
        }
        sw += vw;
        sp += vp;
    }
}

struct P2Shared {
    uint32_t bits[kChunk<1> / 32];
    int last;
};

template <int DT, bool VEC>
__device__ void finalize_pass2(const Pass2Args& a, int sidx, int b, int pos, bool valid, int64_t r, int mode,
                               const WParams& wp, P2Shared& sh) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int lane = lane_id();
    const int nseg = a.nb * kWavesPerBlock;
    const double2* seg = a.seg + (int64_t)sidx * a.seg_stride;
    const int K = a.K;
    int tok = -1;
    double Zused = 0.0;
    if (valid) {
        // totals over segments in segment order (fixed-shape wave scans)
        double tot_w = 0.0, tot_p = 0.0;
        for (int g0 = 0; g0 < nseg; g0 += kWave) {
            const int g = g0 + lane;
            double iw = 0.0, ip = 0.0;
            if (g < nseg) {
                iw = observe(&seg[g].x);
                ip = observe(&seg[g].y);
            }
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const double yw = __shfl_up(iw, off, kWave);
                const double yp = __shfl_up(ip, off, kWave);
                if (lane >= off) {
                    iw += yw;
                    ip += yp;
                }
            }
            tot_w += __shfl(iw, kWave - 1, kWave);
            tot_p += __shfl(ip, kWave - 1, kWave);
        }
        int wmode = mode;
        double Z = tot_w;
        if (mode == kWResid && !(Z > 0.0)) {
            wmode = kWP;
            Z = tot_p;
        }
        Zused = Z;
        const uint32_t purpose = a.mode == 0 ? kPurposeBonus : kPurposeDraft;
        const double u = (double)philox_uniform(a.seed, a.round, purpose, (uint64_t)b, (uint64_t)pos);
        const double t = u * Z;
        // first segment whose inclusive running sum exceeds t
        int gsel = -1, glast = -1;
        double gbase = 0.0, lastbase = 0.0, carry = 0.0;
        for (int g0 = 0; g0 < nseg; g0 += kWave) {
            const int g = g0 + lane;
            double x = 0.0;
            if (g < nseg) x = (wmode == kWP && mode == kWResid) ? observe(&seg[g].y) : observe(&seg[g].x);
            double incl = x;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const double y = __shfl_up(incl, off, kWave);
                if (lane >= off) incl += y;
            }
            incl += carry;
            const double excl = incl - x;
            const uint64_t cross = __ballot(g < nseg && incl > t);
            const uint64_t pos_m = __ballot(g < nseg && x > 0.0);
            if (gsel < 0 && cross) {
                const int l = __ffsll((long long)cross) - 1;
                gsel = g0 + l;
                gbase = __shfl(excl, l, kWave);
            }
            if (pos_m) {
                const int l = 63 - __clzll(pos_m);
                glast = g0 + l;
                lastbase = __shfl(excl, l, kWave);
            }
            carry = __shfl(incl, kWave - 1, kWave);
        }
        bool pick_last = false;
        if (gsel < 0) {
            gsel = glast < 0 ? 0 : glast;
            gbase = lastbase;
            pick_last = true;
        }
        // rescan the selected segment (one wave tile) element by element in id order
        const int64_t c0 = (int64_t)(gsel / kWavesPerBlock) * kChunk<DT>;
        const int64_t tile0 = c0 + (int64_t)(gsel % kWavesPerBlock) * kTile<DT>;
        const int F = a.F[pos];
        const int32_t* ids = a.cache_ids + (int64_t)b * a.Bf + a.O[pos];
        if (wmode != kWP) {
            clear_bitmap<DT>(sh.bits, lane, kWave);
            wave_sync_lds();
            set_bitmap<DT>(sh.bits, c0, ids, F, lane, kWave);
            wave_sync_lds();
        }
        const char* prow = a.p_logits ? a.p_logits + r * a.ld_bytes : nullptr;
        const char* qrow = a.q_logits + r * a.ld_bytes;
        double run = gbase;
        int found = -1, last_pos = -1;
        for (int j = 0; j < kVecPerLane && found < 0; ++j) {
            const int64_t e0 = tile0 + (int64_t)(j * kWave + lane) * N;
            double w[N], p[N];
            u32x4 rp, rq;
            load_pair<DT, VEC>(wmode, prow, qrow, e0, a.V, rp, rq);
            vec_weights<DT>(wmode, wp, rp, rq, e0, a.V, sh.bits, c0, w, p);
            double ls = 0.0;
#pragma unroll
            for (int e = 0; e < N; ++e) ls += w[e];
            double incl = ls;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const double y = __shfl_up(incl, off, kWave);
                if (lane >= off) incl += y;
            }
            double cum = run + (incl - ls);
            int hitpos = -1, lastp = -1;
#pragma unroll
            for (int e = 0; e < N; ++e) {
                cum += w[e];
                if (hitpos < 0 && cum > t) hitpos = (int)(e0 + e);
                if (w[e] > 0.0) lastp = (int)(e0 + e);
            }
            if (!pick_last) {
                const uint64_t hm = __ballot(hitpos >= 0);
                if (hm) found = __shfl(hitpos, __ffsll((long long)hm) - 1, kWave);
            }
            const uint64_t lm = __ballot(lastp >= 0);
            if (lm) last_pos = __shfl(lastp, 63 - __clzll(lm), kWave);
            run += __shfl(incl, kWave - 1, kWave);
        }
        tok = found >= 0 ? found : (last_pos >= 0 ? last_pos : (int)min<int64_t>(tile0, a.V - 1));
    }
    if (lane == 0) {
        if (a.mode == 0) {
            a.out_tok[b] = tok;
            if (a.resid_mass) a.resid_mass[b] = Zused;
            if (!valid && a.dev_err) a.dev_err[b] |= kErrLenRange;
        } else {
            a.out_tok[(int64_t)b * K + pos] = tok;
        }
    }
    if (a.mode == 0 && a.do_lookup)
        lookup_wave(b, K, a.V, valid ? pos : -1, tok, a.F, a.O, a.Bf, a.cache_ids, a.fallback, a.seed, a.round,
                    a.hit, a.slot, a.fallback_tokens);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void pass2_kernel(const Pass2Args a) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    __shared__ P2Shared sh;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int sidx = blockIdx.x / a.nb, blk = blockIdx.x % a.nb;
    const int K = a.K, K1 = K + 1;
    int b, pos;
    bool valid;
    if (a.mode == 0) {
        b = sidx;
        pos = a.accept_len[b];
        valid = pos >= 0 && pos <= K;
    } else {
        b = sidx / K;
        pos = sidx % K;
        valid = true;
    }
    if (!valid) pos = 0;
    const int64_t r = (int64_t)b * K1 + pos;
    const int mode = a.mode == 1 ? kWQprime : (pos < K ? kWResid : kWP);
    const WParams wp = make_wparams(a, r);
    const int64_t c0 = (int64_t)blk * kChunk<DT>;
    const int F = a.F[pos];
    const int32_t* ids = a.cache_ids + (int64_t)b * a.Bf + a.O[pos];
    if (mode != kWP) {
        clear_bitmap<DT>(sh.bits, tid, kBlock);
        __syncthreads();
        set_bitmap<DT>(sh.bits, c0, ids, F, tid, kBlock);
    }
    __syncthreads();

    const char* prow = a.p_logits ? a.p_logits + r * a.ld_bytes : nullptr;
    const char* qrow = a.q_logits + r * a.ld_bytes;
    const int64_t tile0 = c0 + (int64_t)wave * kTile<DT>;
    double sw = 0.0, sp = 0.0;
    if (valid) {
        if (mode == kWResid)
            tile_sums<DT, VEC, kWResid>(wp, prow, qrow, tile0, a.V, sh.bits, c0, sw, sp);
        else if (mode == kWP)
            tile_sums<DT, VEC, kWP>(wp, prow, qrow, tile0, a.V, sh.bits, c0, sw, sp);
        else
            tile_sums<DT, VEC, kWQprime>(wp, prow, qrow, tile0, a.V, sh.bits, c0, sw, sp);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        sw += __shfl_xor(sw, m, kWave);
        sp += __shfl_xor(sp, m, kWave);
    }
    if (lane == 0) {
        double2* g = a.seg + (int64_t)sidx * a.seg_stride + blk * kWavesPerBlock + wave;
        publish(&g->x, sw);
        publish(&g->y, sp);
    }

    wait_stores();
    __syncthreads();
    if (tid == 0) {
        const unsigned old = arrive(&a.counter[sidx]);
        sh.last = (old == (unsigned)a.nb - 1u);
        if (sh.last) publish(&a.counter[sidx], 0u);
    }
    __syncthreads();
    if (!sh.last) return;
    if (wave != 0) return;
    finalize_pass2<DT, VEC>(a, sidx, b, pos, valid, r, mode, wp, sh);
}

// ============================================================================ small kernels
__global__ void combine_stats_kernel(const Pass1Args a, float* m_out, double* s_out, int32_t* arg_out) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= a.B * a.K1) return;
    const int b = r / a.K1, i = r % a.K1;
    float m;
    double s;
    int arg;
    combine_partials(a.part + (int64_t)b * a.part_stride + (int64_t)i * a.nb, a.nb, a.c, m, s, arg);
    m_out[r] = m;
    s_out[r] = a.greedy ? 1.0 : std_sum(m, s, a.c);
    if (arg_out) arg_out[r] = arg;
}

__global__ __launch_bounds__(kBlock) void combine_topf_kernel(const Pass1Args a, int Bf, const float* q_max,
                                                              const double* q_sum, int32_t* cache_ids,
                                                              double* cache_mass) {
    __shared__ uint64_t xchg[kWavesPerBlock][kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (r >= (int64_t)a.B * a.K1) return;
    const int b = (int)(r / a.K1), i = (int)(r % a.K1);
    const double M = cache_row(a.topk + (int64_t)b * a.topk_stride + (int64_t)i * a.nb * a.Fmax, a.nb, a.Fmax, a.F[i],
                               q_max[r], q_sum[r], a.c, a.greedy, cache_ids + (int64_t)b * Bf + a.O[i], nullptr,
                               xchg[wave]);
    if (lane == 0) cache_mass[r] = M;
}

struct FO {
    int F[kMaxK + 1];
    int O[kMaxK + 2];
};

template <int DT>
__global__ void probs_kernel(const char* logits, int B, int K1, int V, int64_t ld_bytes, const float* m,
                             const double* s, const int32_t* arg, float c, int greedy, const int32_t* cache_ids, FO fo,
                             int Bf, const double* Z, float C, float* out) {
    const int64_t r = blockIdx.y;
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= V) return;
    const int b = (int)(r / K1), i = (int)(r % K1);
    double p;
    if (greedy) {
        p = (x == arg[r]) ? 1.0 : 0.0;
    } else {
        const RowNorm n = row_norm(m[r], s[r], c);
        p = (double)term(load_one<DT>(logits + r * ld_bytes, x), c, n.o) * n.inv;
    }
    if (Z) {
        bool in_cache = false;
        const int32_t* ids = cache_ids + (int64_t)b * Bf + fo.O[i];
        for (int j = 0; j < fo.F[i]; ++j) in_cache |= ids[j] == (int32_t)x;
        p = p * (in_cache ? (double)C : 1.0) / Z[r];
    }
    out[r * V + x] = (float)p;
}

__global__ void saguaro_z_kernel(const double* mass, int R, float C, double* Z) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r < R) Z[r] = 1.0 - (1.0 - (double)C) * mass[r];
}

template <int DT>
__global__ void verify_kernel(const char* p_logits, const char* q_logits, int B, int K, int V, int64_t ld_bytes,
                              const int32_t* draft, const float* p_max, const double* p_sum, const int32_t* p_arg,
                              const float* q_max, const double* q_sum, FO fo, int Bf, const int32_t* cache_ids,
                              const double* Z, float C, float c, int greedy, uint64_t seed, uint64_t round,
                              int32_t* accept_len, float* accept_prob, int32_t* dev_err) {
    const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const int lane = lane_id();
    const int K1 = K + 1;
    const bool act = lane < K;
    const int ic = act ? lane : 0;
    const int64_t r = (int64_t)b * K1 + ic;
    const int d = act ? draft[(int64_t)b * K + lane] : 0;
    bool in_cache = false;
    const int32_t* ids = cache_ids + (int64_t)b * Bf + fo.O[ic];
    for (int j = 0; j < fo.F[ic]; ++j) in_cache |= ids[j] == d;
    const float mp = greedy ? 0.f : p_max[r], mq = greedy ? 0.f : q_max[r];
    const double sp = greedy ? 1.0 : p_sum[r], sq = greedy ? 1.0 : q_sum[r];
    const int argp = greedy ? p_arg[r] : 0;
    const double Zi = greedy ? 1.0 : Z[r];
    int errs;
    const int k = verify_wave<DT>(b, K, V, p_logits + r * ld_bytes, q_logits + r * ld_bytes, d, mp, sp, argp, mq, sq,
                                  Zi, in_cache, C, c, greedy, seed, round, accept_prob, &errs);
    if (lane == 0) {
        accept_len[b] = k;
        if (dev_err && errs) dev_err[b] |= errs;
    }
}

__global__ void greedy_pick_kernel(const int32_t* arg, int B, int K, const int32_t* accept_len, int32_t* out,
                                   double* mass, int32_t* dev_err) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int K1 = K + 1;
    if (!accept_len) {
        if (t >= B * K) return;
        const int b = t / K, i = t % K;
        out[t] = arg[(int64_t)b * K1 + i];
    } else {
        if (t >= B) return;
        const int k = accept_len[t];
        const bool ok = k >= 0 && k <= K;
        out[t] = ok ? arg[(int64_t)t * K1 + k] : -1;
        if (mass) mass[t] = ok ? 1.0 : 0.0;
        if (!ok && dev_err) dev_err[t] |= kErrLenRange;
    }
}

__global__ void lookup_kernel(int B, int K, int V, FO fo, int Bf, const int32_t* cache_ids, const int32_t* accept_len,
                              const int32_t* bonus, int fallback, uint64_t seed, uint64_t round, uint8_t* hit,
                              int32_t* slot, int32_t* fb, int32_t* dev_err) {
    const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const int k = accept_len[b];
    const bool ok = k >= 0 && k <= K;
    if (!ok && lane_id() == 0 && dev_err) dev_err[b] |= kErrLenRange;
    lookup_wave(b, K, V, ok ? k : -1, bonus[b], fo.F, fo.O, Bf, cache_ids, fallback, seed, round, hit, slot, fb);
}

// ============================================================================ launchers
static FO make_fo(const int* F, const int* O, int K1) {
    FO fo;
    for (int i = 0; i <= kMaxK; ++i) fo.F[i] = i < K1 ? F[i] : 0;
    for (int i = 0; i <= kMaxK + 1; ++i) fo.O[i] = i <= K1 ? O[i] : 0;
    return fo;
}

hipError_t launch_pass1(int dtype, bool vec, const Pass1Args& a, hipStream_t st) {
    const int64_t grid = (int64_t)a.B * a.nmodel * a.K1 * a.nb;
    if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
    if (dtype == 1) {
        if (vec)
            pass1_kernel<1, true><<<(unsigned)grid, kBlock, 0, st>>>(a);
        else
            pass1_kernel<1, false><<<(unsigned)grid, kBlock, 0, st>>>(a);
    } else {
        if (vec)
            pass1_kernel<0, true><<<(unsigned)grid, kBlock, 0, st>>>(a);
        else
            pass1_kernel<0, false><<<(unsigned)grid, kBlock, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_pass2(int dtype, bool vec, const Pass2Args& a, int nseq, hipStream_t st) {
    const int64_t grid = (int64_t)nseq * a.nb;
    if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
    if (dtype == 1) {
        if (vec)
            pass2_kernel<1, true><<<(unsigned)grid, kBlock, 0, st>>>(a);
        else
            pass2_kernel<1, false><<<(unsigned)grid, kBlock, 0, st>>>(a);
    } else {
        if (vec)
            pass2_kernel<0, true><<<(unsigned)grid, kBlock, 0, st>>>(a);
        else
            pass2_kernel<0, false><<<(unsigned)grid, kBlock, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_combine_stats(const Pass1Args& a, float* m, double* s, int32_t* arg, hipStream_t st) {
    const int R = a.B * a.K1;
    combine_stats_kernel<<<(R + 255) / 256, 256, 0, st>>>(a, m, s, arg);
    return hipGetLastError();
}

hipError_t launch_combine_topf(const Pass1Args& a, int Bf, const float* q_max, const double* q_sum,
                               int32_t* cache_ids, double* cache_mass, hipStream_t st) {
    const int R = a.B * a.K1;
    combine_topf_kernel<<<(R + kWavesPerBlock - 1) / kWavesPerBlock, kBlock, 0, st>>>(a, Bf, q_max, q_sum, cache_ids,
                                                                                      cache_mass);
    return hipGetLastError();
}

hipError_t launch_probs(int dtype, const char* logits, int B, int K1, int V, int64_t ld_bytes, const float* m,
                        const double* s, const int32_t* arg, float c, int greedy, const int32_t* cache_ids,
                        const int* F, const int* O, int Bf, const double* Z, float C, float* out, hipStream_t st) {
    dim3 grid((V + 255) / 256, B * K1);
    FO fo = F ? make_fo(F, O, K1) : FO{};
    if (dtype == 1)
        probs_kernel<1><<<grid, 256, 0, st>>>(logits, B, K1, V, ld_bytes, m, s, arg, c, greedy, cache_ids, fo, Bf, Z,
                                              C, out);
    else
        probs_kernel<0><<<grid, 256, 0, st>>>(logits, B, K1, V, ld_bytes, m, s, arg, c, greedy, cache_ids, fo, Bf, Z,
                                              C, out);
    return hipGetLastError();
}

hipError_t launch_saguaro_z(const double* cache_mass, int R, float C, double* Z, hipStream_t st) {
    saguaro_z_kernel<<<(R + 255) / 256, 256, 0, st>>>(cache_mass, R, C, Z);
    return hipGetLastError();
}

hipError_t launch_verify(int dtype, const char* p_logits, const char* q_logits, int B, int K, int V,
                         int64_t ld_bytes, const int32_t* draft, const float* p_max, const double* p_sum,
                         const int32_t* p_arg, const float* q_max, const double* q_sum, const int* F, const int* O,
                         int Bf, const int32_t* cache_ids, const double* Z, float C, float c, int greedy,
                         uint64_t seed, uint64_t round, int32_t* accept_len, float* accept_prob, int32_t* dev_err,
                         hipStream_t st) {
    const int per_block = kWavesPerBlock;
    const FO fo = make_fo(F, O, K + 1);
    if (dtype == 1)
        verify_kernel<1><<<(B + per_block - 1) / per_block, kBlock, 0, st>>>(
            p_logits, q_logits, B, K, V, ld_bytes, draft, p_max, p_sum, p_arg, q_max, q_sum, fo, Bf, cache_ids, Z, C,
            c, greedy, seed, round, accept_len, accept_prob, dev_err);
    else
        verify_kernel<0><<<(B + per_block - 1) / per_block, kBlock, 0, st>>>(
            p_logits, q_logits, B, K, V, ld_bytes, draft, p_max, p_sum, p_arg, q_max, q_sum, fo, Bf, cache_ids, Z, C,
            c, greedy, seed, round, accept_len, accept_prob, dev_err);
    return hipGetLastError();
}

hipError_t launch_greedy_pick(const int32_t* arg, int B, int K, const int32_t* accept_len, int32_t* out, double* mass,
                              int32_t* dev_err, hipStream_t st) {
    const int n = accept_len ? B : B * K;
    greedy_pick_kernel<<<(n + 255) / 256, 256, 0, st>>>(arg, B, K, accept_len, out, mass, dev_err);
    return hipGetLastError();
}

hipError_t launch_lookup(int B, int K, int V, const int* F, const int* O, int Bf, const int32_t* cache_ids,
                         const int32_t* accept_len, const int32_t* bonus, int fallback, uint64_t seed,
                         uint64_t round, uint8_t* hit, int32_t* slot, int32_t* fallback_tokens, int32_t* dev_err,
                         hipStream_t st) {
    const FO fo = make_fo(F, O, K + 1);
    lookup_kernel<<<(B + kWavesPerBlock - 1) / kWavesPerBlock, kBlock, 0, st>>>(
        B, K, V, fo, Bf, cache_ids, accept_len, bonus, fallback, seed, round, hit, slot, fallback_tokens, dev_err);
    return hipGetLastError();
}

}  // namespace ssd
