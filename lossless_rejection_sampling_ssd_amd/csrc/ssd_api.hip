// ssd_api.hip -- the C ABI (include/ssd.h): host-side validation, workspace layout
// and kernel launches.  No allocation, no synchronisation; the only state is the
// per-GPU address of the no-allocation round's static scratch array.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/ssd.h"
#include "ssd_kernels.h"
#include "ssd_ngram.h"

namespace {

// Text of the last HIP failure of this thread; a fixed buffer, so that recording it
// can neither allocate nor throw across the C ABI.
thread_local char g_last_error[256];

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace regions (byte offsets).  Every region is written by one kernel of a call
// and read by a later kernel of the same call; nothing persists between calls.
//   part   [B][2][K+1][nt]        WavePartial, one per wave tile
//   cand   [B][K+1][nu][4 cap]    top-F candidate keys of the draft rows, per unit of four
//                                 tiles (nu = ceil(nt / 4))
//   seg    [max(B, B K)][nt2]     (weight sum, target-law sum) per pass-2 tile
//   stats  [B (K+1)]              fp64 p_sum q_sum cache_mass Z, fp32 p_max q_max,
//                                 int32 p_arg (for outputs the caller leaves NULL)
//   vflag  [B K]                  int32 outcome of each draft-token test
//   probe  [B K 2]                fp32 logits at the draft tokens (target, draft)
//   law    [B (K+1)]              LawParams of each row (fused round: written by the
//                                 finalisation, read by pass 2 and the bonus)
struct Layout {
    size_t part, cand, seg, stats, vflag, probe, law, total;
    int nt, nt2, cap;
};

void layout_for(const ssd_shape* s, int32_t Bf, Layout* L) {
    const int64_t K1 = s->K + 1;
    const int64_t R = (int64_t)s->B * K1;
    const int nt = ssd::tiles_per_row(s->dtype, s->V);
    const int nt2 = ssd::tiles_per_row2(s->dtype, s->V);
    const int Fmax = Bf < 1 ? 1 : (Bf > SSD_MAX_F ? SSD_MAX_F : Bf);
    const int cap = ssd::cand_cap(Fmax);
    const int64_t groups = std::max<int64_t>(s->B, (int64_t)s->B * s->K);
    size_t off = 0;
    L->part = off;
    off = align_up(off + (size_t)R * 2 * nt * sizeof(ssd::WavePartial));
    L->cand = off;
    // keys per unit of four tiles (one pass-1 block), 4 cap slots each
    off = align_up(off + (size_t)R * ((nt + 3) / 4) * 4 * cap * sizeof(uint64_t));
    L->seg = off;
    off = align_up(off + (size_t)groups * nt2 * 16);
    L->stats = off;
    off = align_up(off + (size_t)R * (4 * 8 + 2 * 4 + 4));
    L->vflag = off;
    off = align_up(off + (size_t)s->B * s->K * 4);
    L->probe = off;
    off = align_up(off + (size_t)s->B * s->K * 8);
    L->law = off;
    off = align_up(off + (size_t)R * sizeof(ssd::LawParams));
    L->total = off;
    L->nt = nt;
    L->nt2 = nt2;
    L->cap = cap;
}

ssd_status fail_hip(hipError_t e, const char* where) {
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
    return SSD_ERR_HIP;
}

ssd_status check_shape(const ssd_shape* s) {
    if (!s) return SSD_ERR_ARG;
    if (s->B < 1 || s->K < 1 || s->K > SSD_MAX_K || s->V < 2 || s->ld < s->V) return SSD_ERR_ARG;
    if (s->dtype != SSD_F32 && s->dtype != SSD_BF16) return SSD_ERR_ARG;
    if (!std::isfinite(s->T) || s->T < 0.f) return SSD_ERR_ARG;
    const int64_t nt = ssd::tiles_per_row(s->dtype, s->V), nt2 = ssd::tiles_per_row2(s->dtype, s->V);
    const int64_t grid1 = ((int64_t)s->B * (s->K + 1) + 7) / 8 * 8 * 2 * ((nt + 3) / 4);
    const int64_t grid2 = (int64_t)s->B * s->K * ((nt2 + 3) / 4);
    if (grid1 > 0x7FFFFFFF || grid2 > 0x7FFFFFFF) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd_status check_fanout(const ssd_shape* s, const int32_t* F, int32_t Bf, int* O) {
    if (!F || Bf < 0) return SSD_ERR_ARG;
    int64_t sum = 0;
    O[0] = 0;
    for (int k = 0; k <= s->K; ++k) {
        if (F[k] < 0 || F[k] > s->V) return SSD_ERR_ARG;
        sum += F[k];
        O[k + 1] = (int)sum;
    }
    if (sum != Bf) return SSD_ERR_ARG;
    for (int k = 0; k <= s->K; ++k)
        if (F[k] > SSD_MAX_F) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd_status check_ws(const ssd_shape* s, int32_t Bf, void* ws, size_t ws_bytes, Layout* L) {
    layout_for(s, Bf, L);
    if (!ws || ((uintptr_t)ws % kAlign) != 0) return SSD_ERR_ARG;
    if (ws_bytes < L->total) return SSD_ERR_WORKSPACE;
    return SSD_OK;
}

bool vec_ok(const ssd_shape* s, const void* p) {
    const int es = s->dtype == SSD_BF16 ? 2 : 4;
    return p && ((uintptr_t)p % 16 == 0) && ((s->ld * es) % 16 == 0);
}

float temp_scale(float T) { return T > 0.f ? (float)(1.4426950408889634 / (double)T) : 0.f; }

int64_t ld_bytes(const ssd_shape* s) { return s->ld * (s->dtype == SSD_BF16 ? 2 : 4); }

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

void fill_fo(ssd::Pass1Args& a, const int32_t* F, const int* O, int K1) {
    for (int i = 0; i <= ssd::kMaxKc; ++i) a.F[i] = i < K1 ? F[i] : 0;
    for (int i = 0; i <= ssd::kMaxKc + 1; ++i) a.O[i] = i <= K1 ? O[i] : 0;
}
void fill_fo(ssd::Pass2Args& a, const int32_t* F, const int* O, int K1) {
    for (int i = 0; i <= ssd::kMaxKc; ++i) a.F[i] = i < K1 ? F[i] : 0;
    for (int i = 0; i <= ssd::kMaxKc + 1; ++i) a.O[i] = i <= K1 ? O[i] : 0;
}

int zeros_F[SSD_MAX_K + 1] = {0};

// Scratch of ssd_round_noalloc: one copy per GPU, looked up once per device.  In host
// code `scratch` names a host-side stand-in, never the device memory: only the
// address hipGetSymbolAddress returns (kept in g_scratch) is handed to kernels.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

void set_ws(ssd::Pass1Args& a, void* ws, const Layout& L) {
    a.nt = L.nt;
    a.cap = L.cap;
    a.part = at<ssd::WavePartial>(ws, L.part);
    a.cand = at<uint64_t>(ws, L.cand);
}

}  // namespace

static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

// The device address of this GPU's copy of `scratch` (the device of `stream`, or the
// current one for the null stream), looked up on the first call on that GPU.
ssd_status scratch_for(hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "ssd_round_noalloc device");
    if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = -1;
            if ((e = hipGetDevice(&cur)) != hipSuccess) return fail_hip(e, "ssd_round_noalloc device");
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return fail_hip(e, "ssd_round_noalloc device");
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
            if (e != hipSuccess) return fail_hip(e, "ssd_round_noalloc scratch lookup");
            if (e2 != hipSuccess) return fail_hip(e2, "ssd_round_noalloc device");
            if (!p || ((uintptr_t)p % kAlign) != 0) {
                snprintf(g_last_error, sizeof(g_last_error), "ssd_round_noalloc: scratch address %p unusable", p);
                return SSD_ERR_HIP;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SSD_OK;
}

}  // namespace

extern "C" {

const char* ssd_status_string(ssd_status s) {
    switch (s) {
        case SSD_OK: return "ok";
        case SSD_ERR_ARG: return "invalid argument";
        case SSD_ERR_UNSUPPORTED: return "unsupported shape";
        case SSD_ERR_HIP: return "HIP error";
        case SSD_ERR_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

const char* ssd_last_error(void) { return g_last_error; }

ssd_status ssd_fanout(int32_t K, int32_t Bf, double r, int32_t* F_host) {
    if (!F_host || K < 1 || K > SSD_MAX_K || Bf < 0 || !(r > 0.0) || !(r <= 1.0)) return SSD_ERR_ARG;
    double w[SSD_MAX_K + 1], sum = 0.0, x = 1.0;
    for (int k = 0; k <= K; ++k) {
        w[k] = x;
        sum += x;
        x *= r;
    }
    double rem[SSD_MAX_K + 1];
    bool up[SSD_MAX_K + 1];
    int given = 0;
    for (int k = 0; k <= K; ++k) {
        const double share = (double)Bf * w[k] / sum;
        const double fl = std::floor(share);
        F_host[k] = (int32_t)fl;
        rem[k] = share - fl;
        up[k] = false;
        given += F_host[k];
    }
    for (int left = Bf - given; left > 0; --left) {
        int best = -1;
        for (int k = 0; k <= K; ++k)
            if (!up[k] && (best < 0 || rem[k] > rem[best])) best = k;
        up[best] = true;
        F_host[best] += 1;
    }
    return SSD_OK;
}

size_t ssd_workspace_bytes(const ssd_shape* shape, int32_t Bf) {
    if (check_shape(shape) != SSD_OK) return 0;
    Layout L;
    layout_for(shape, Bf, &L);
    return L.total;
}

ssd_status ssd_softmax(const ssd_shape* s, const void* logits, float* row_max, double* row_sum,
                       int32_t* row_argmax, float* probs, void* ws, size_t ws_bytes, void* stream) {
    ssd_status st = check_shape(s);
    if (st != SSD_OK) return st;
    if (!logits || !row_max || !row_sum) return SSD_ERR_ARG;
    Layout L;
    if ((st = check_ws(s, 1, ws, ws_bytes, &L)) != SSD_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    const int K1 = s->K + 1, R = s->B * K1;
    if (probs && R > 65535) return SSD_ERR_UNSUPPORTED;  // dense output: one grid row per logit row
    const int greedy = s->T == 0.f;
    ssd::Pass1Args a{};
    a.logits[0] = (const char*)logits;
    a.logits[1] = nullptr;
    a.nmodel = 1;
    a.topf_model = -1;
    a.B = s->B;
    a.K1 = K1;
    a.V = s->V;
    a.ld_bytes = ld_bytes(s);
    a.c = temp_scale(s->T);
    a.greedy = greedy;
    a.want_arg = greedy || row_argmax != nullptr || probs != nullptr;
    int O[SSD_MAX_K + 2] = {0};
    fill_fo(a, zeros_F, O, K1);
    set_ws(a, ws, L);
    hipError_t e = ssd::launch_pass1(s->dtype, vec_ok(s, logits), a, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_softmax pass");
    int32_t* argp = row_argmax ? row_argmax : at<int32_t>(ws, L.stats);
    e = ssd::launch_combine_stats(a, row_max, row_sum, argp, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_softmax combine");
    if (probs) {
        e = ssd::launch_probs(s->dtype, (const char*)logits, s->B, K1, s->V, a.ld_bytes, row_max, row_sum, argp, a.c,
                              greedy, nullptr, nullptr, nullptr, 0, nullptr, 1.f, probs, hs);
        if (e != hipSuccess) return fail_hip(e, "ssd_softmax probs");
    }
    return SSD_OK;
}

ssd_status ssd_build_cache(const ssd_shape* s, const void* q_logits, const float* q_max, const double* q_sum,
                           const int32_t* F_host, int32_t Bf, int32_t* cache_ids, double* cache_mass, void* ws,
                           size_t ws_bytes, void* stream) {
    ssd_status st = check_shape(s);
    if (st != SSD_OK) return st;
    int O[SSD_MAX_K + 2];
    if ((st = check_fanout(s, F_host, Bf, O)) != SSD_OK) return st;
    if (!q_logits || !q_max || !q_sum || !cache_mass || (Bf > 0 && !cache_ids)) return SSD_ERR_ARG;
    Layout L;
    if ((st = check_ws(s, Bf, ws, ws_bytes, &L)) != SSD_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    const int K1 = s->K + 1;
    const int greedy = s->T == 0.f;
    ssd::Pass1Args a{};
    a.logits[0] = (const char*)q_logits;
    a.nmodel = 1;
    a.topf_model = 0;
    a.B = s->B;
    a.K1 = K1;
    a.V = s->V;
    a.ld_bytes = ld_bytes(s);
    a.c = temp_scale(s->T);
    a.greedy = greedy;
    a.want_arg = 0;
    fill_fo(a, F_host, O, K1);
    set_ws(a, ws, L);
    hipError_t e = ssd::launch_pass1(s->dtype, vec_ok(s, q_logits), a, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_build_cache pass");
    e = ssd::launch_combine_topf(a, Bf, q_max, q_sum, cache_ids, cache_mass, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_build_cache combine");
    return SSD_OK;
}

ssd_status ssd_saguaro_reweight(const ssd_shape* s, const double* cache_mass, float C, double* Z,
                                const void* q_logits, const float* q_max, const double* q_sum, const int32_t* q_argmax,
                                const int32_t* F_host, int32_t Bf, const int32_t* cache_ids, float* q_prime,
                                ssd_rng rng, int32_t* draft, void* ws, size_t ws_bytes, void* stream) {
    ssd_status st = check_shape(s);
    if (st != SSD_OK) return st;
    if (!cache_mass || !Z || !(C > 0.f) || !(C <= 1.f)) return SSD_ERR_ARG;
    const int K1 = s->K + 1, R = s->B * K1;
    const int greedy = s->T == 0.f;
    int O[SSD_MAX_K + 2] = {0};
    const bool extra = q_prime || draft;
    Layout L;
    if (extra) {
        if ((st = check_fanout(s, F_host, Bf, O)) != SSD_OK) return st;
        if (!q_logits || !q_max || !q_sum || (Bf > 0 && !cache_ids)) return SSD_ERR_ARG;
        if (greedy && !q_argmax) return SSD_ERR_ARG;
        if (draft && (st = check_ws(s, Bf, ws, ws_bytes, &L)) != SSD_OK) return st;
    }
    if (q_prime && R > 65535) return SSD_ERR_UNSUPPORTED;  // dense output: one grid row per logit row
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = ssd::launch_saguaro_z(cache_mass, R, C, Z, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_saguaro_reweight Z");
    const float c = temp_scale(s->T);
    if (q_prime) {
        e = ssd::launch_probs(s->dtype, (const char*)q_logits, s->B, K1, s->V, ld_bytes(s), q_max, q_sum, q_argmax, c,
                              greedy, cache_ids, F_host, O, Bf, Z, C, q_prime, hs);
        if (e != hipSuccess) return fail_hip(e, "ssd_saguaro_reweight q'");
    }
    if (draft) {
        if (greedy) {
            e = ssd::launch_greedy_pick(q_argmax, s->B, s->K, nullptr, draft, nullptr, nullptr, hs);
        } else {
            ssd::Pass2Args a{};
            a.p_logits = nullptr;
            a.q_logits = (const char*)q_logits;
            a.B = s->B;
            a.K = s->K;
            a.V = s->V;
            a.ld_bytes = ld_bytes(s);
            a.c = c;
            a.C = C;
            a.mode = 1;
            a.nt = L.nt2;
            fill_fo(a, F_host, O, K1);
            a.Bf = Bf;
            a.q_max = q_max;
            a.q_sum = q_sum;
            a.Z = Z;
            a.cache_ids = cache_ids;
            a.seed = rng.seed;
            a.round = rng.round;
            a.seg = at<double2>(ws, L.seg);
            a.out_tok = draft;
            const bool vec = vec_ok(s, q_logits);
            e = ssd::launch_pass2(s->dtype, vec, a, s->B * s->K, hs);
            if (e == hipSuccess) e = ssd::launch_finalize_bonus(s->dtype, vec, a, s->B * s->K, hs);
        }
        if (e != hipSuccess) return fail_hip(e, "ssd_saguaro_reweight draft");
    }
    return SSD_OK;
}

ssd_status ssd_verify(const ssd_shape* s, const void* p_logits, const void* q_logits, const int32_t* draft,
                      const float* p_max, const double* p_sum, const int32_t* p_argmax, const float* q_max,
                      const double* q_sum, const int32_t* F_host, int32_t Bf, const int32_t* cache_ids, const double* Z,
                      float C, ssd_rng rng, int32_t* accept_len, float* accept_prob, int32_t* dev_err,
                      void* stream) {
    ssd_status st = check_shape(s);
    if (st != SSD_OK) return st;
    int O[SSD_MAX_K + 2];
    if ((st = check_fanout(s, F_host, Bf, O)) != SSD_OK) return st;
    const int greedy = s->T == 0.f;
    if (!draft || !accept_len || !(C > 0.f) || !(C <= 1.f)) return SSD_ERR_ARG;
    // the membership test of d_i reads the cached ids at every temperature
    if (Bf > 0 && !cache_ids) return SSD_ERR_ARG;
    if (greedy && !p_argmax) return SSD_ERR_ARG;
    if (!greedy && (!p_logits || !q_logits || !p_max || !p_sum || !q_max || !q_sum || !Z)) return SSD_ERR_ARG;
    hipError_t e = ssd::launch_verify(s->dtype, (const char*)p_logits, (const char*)q_logits, s->B, s->K, s->V,
                                      ld_bytes(s), draft, p_max, p_sum, p_argmax, q_max, q_sum, F_host, O, Bf,
                                      cache_ids, Z, C, temp_scale(s->T), greedy, rng.seed, rng.round, accept_len,
                                      accept_prob, dev_err, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "ssd_verify");
    return SSD_OK;
}

ssd_status ssd_residual_sample(const ssd_shape* s, const void* p_logits, const void* q_logits, const float* p_max,
                               const double* p_sum, const int32_t* p_argmax, const float* q_max, const double* q_sum,
                               const int32_t* F_host, int32_t Bf, const int32_t* cache_ids, const double* Z, float C,
                               const int32_t* accept_len, ssd_rng rng, int32_t* bonus, double* resid_mass,
                               int32_t* dev_err, void* ws, size_t ws_bytes, void* stream) {
    ssd_status st = check_shape(s);
    if (st != SSD_OK) return st;
    int O[SSD_MAX_K + 2];
    if ((st = check_fanout(s, F_host, Bf, O)) != SSD_OK) return st;
    const int greedy = s->T == 0.f;
    if (!accept_len || !bonus || !(C > 0.f) || !(C <= 1.f)) return SSD_ERR_ARG;
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e;
    if (greedy) {
        if (!p_argmax) return SSD_ERR_ARG;
        e = ssd::launch_greedy_pick(p_argmax, s->B, s->K, accept_len, bonus, resid_mass, dev_err, hs);
        if (e != hipSuccess) return fail_hip(e, "ssd_residual_sample");
        return SSD_OK;
    }
    if (!p_logits || !q_logits || !p_max || !p_sum || !q_max || !q_sum || !Z || (Bf > 0 && !cache_ids))
        return SSD_ERR_ARG;
    Layout L;
    if ((st = check_ws(s, Bf, ws, ws_bytes, &L)) != SSD_OK) return st;
    ssd::Pass2Args a{};
    a.p_logits = (const char*)p_logits;
    a.q_logits = (const char*)q_logits;
    a.B = s->B;
    a.K = s->K;
    a.V = s->V;
    a.ld_bytes = ld_bytes(s);
    a.c = temp_scale(s->T);
    a.C = C;
    a.mode = 0;
    a.nt = L.nt2;
    fill_fo(a, F_host, O, s->K + 1);
    a.Bf = Bf;
    a.p_max = p_max;
    a.p_sum = p_sum;
    a.q_max = q_max;
    a.q_sum = q_sum;
    a.Z = Z;
    a.cache_ids = cache_ids;
    a.accept_len = accept_len;
    a.seed = rng.seed;
    a.round = rng.round;
    a.seg = at<double2>(ws, L.seg);
    a.out_tok = bonus;
    a.resid_mass = resid_mass;
    a.dev_err = dev_err;
    a.do_lookup = 0;
    const bool vec = vec_ok(s, p_logits) && vec_ok(s, q_logits);
    e = ssd::launch_pass2(s->dtype, vec, a, s->B, hs);
    if (e == hipSuccess) e = ssd::launch_finalize_bonus(s->dtype, vec, a, s->B, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_residual_sample");
    return SSD_OK;
}

ssd_status ssd_cache_lookup(int32_t B, int32_t K, int32_t V, const int32_t* F_host, int32_t Bf,
                            const int32_t* cache_ids, const int32_t* accept_len, const int32_t* bonus,
                            int32_t fallback, ssd_rng rng, uint8_t* hit, int32_t* slot, int32_t* fallback_tokens,
                            int32_t* dev_err, void* stream) {
    ssd_shape s{B, K, V, V, SSD_F32, 1.f};
    ssd_status st = check_shape(&s);
    if (st != SSD_OK) return st;
    int O[SSD_MAX_K + 2];
    if ((st = check_fanout(&s, F_host, Bf, O)) != SSD_OK) return st;
    if ((Bf > 0 && !cache_ids) || !accept_len || !bonus || !hit || !slot || !fallback_tokens) return SSD_ERR_ARG;
    if (fallback != SSD_FALLBACK_NONE && fallback != SSD_FALLBACK_UNIFORM) return SSD_ERR_ARG;
    hipError_t e = ssd::launch_lookup(B, K, V, F_host, O, Bf, cache_ids, accept_len, bonus, fallback, rng.seed,
                                      rng.round, hit, slot, fallback_tokens, dev_err, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "ssd_cache_lookup");
    return SSD_OK;
}

ssd_status ssd_bonus_rank(const ssd_shape* s, const void* q_logits, const int32_t* accept_len,
                          const int32_t* bonus, int32_t R, int32_t* rank_out, uint32_t* rank_hist, void* ws,
                          size_t ws_bytes, void* stream) {
    ssd_status st = check_shape(s);
    if (st != SSD_OK) return st;
    if (!q_logits || !accept_len || !bonus || (!rank_out && !rank_hist) || R < 1 || R > SSD_MAX_F)
        return SSD_ERR_ARG;
    Layout L;
    if ((st = check_ws(s, 1, ws, ws_bytes, &L)) != SSD_OK) return st;
    ssd::RankArgs a{};
    a.q_logits = static_cast<const char*>(q_logits);
    a.B = s->B;
    a.K = s->K;
    a.V = s->V;
    a.ld_bytes = ld_bytes(s);
    a.nt = L.nt;
    a.accept_len = accept_len;
    a.bonus = bonus;
    a.counts = at<uint32_t>(ws, L.part);  // B nt words: far below the pass-1 partials region
    a.R = R;
    a.rank_out = rank_out;
    a.hist = rank_hist;
    hipError_t e = ssd::launch_rank(s->dtype, vec_ok(s, q_logits), a, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "ssd_bonus_rank");
    return SSD_OK;
}

ssd_status ssd_cache_gather(int32_t B, int32_t K, int32_t Bf, const int32_t* values, const uint8_t* hit,
                            const int32_t* slot, const int32_t* fallback_tokens, int32_t* next_draft,
                            int32_t* dev_err, void* stream) {
    if (B < 1 || K < 1 || K > SSD_MAX_K || Bf < 0) return SSD_ERR_ARG;
    if ((Bf > 0 && !values) || !hit || !slot || !fallback_tokens || !next_draft) return SSD_ERR_ARG;
    if ((int64_t)B * K > 0x7FFFFFFFLL) return SSD_ERR_UNSUPPORTED;  // one thread per token, 32-bit grid
    hipError_t e = ssd::launch_gather(B, K, Bf, values, hit, slot, fallback_tokens, next_draft, dev_err,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "ssd_cache_gather");
    return SSD_OK;
}

ssd_status ssd_ngram_fallback(int32_t B, int32_t K, int32_t V, const int32_t* hist, int64_t ld_hist,
                              const int32_t* hist_len, const int32_t* draft, const int32_t* accept_len,
                              const int32_t* bonus, const uint8_t* hit, int32_t n_min, int32_t n_max,
                              ssd_rng rng, int32_t* fallback_tokens, int32_t* next_draft, int32_t* match_n,
                              int32_t* match_end, int32_t* dev_err, void* stream) {
    if (B < 1 || K < 1 || K > SSD_MAX_K || V < 2 || ld_hist < 0) return SSD_ERR_ARG;
    if (n_min < 1 || n_max < n_min || n_max > SSD_MAX_NGRAM) return SSD_ERR_ARG;
    if ((ld_hist > 0 && !hist) || !hist_len || !draft || !accept_len || !bonus || !fallback_tokens)
        return SSD_ERR_ARG;
    // context positions (history + K + 1) are 32-bit in the kernel
    if (ld_hist > (int64_t)INT32_MAX - SSD_MAX_K - 1) return SSD_ERR_UNSUPPORTED;
    ssd::NgramArgs a{};
    a.B = B;
    a.K = K;
    a.V = V;
    a.hist = hist;
    a.ld_hist = ld_hist;
    a.hist_len = hist_len;
    a.draft = draft;
    a.accept_len = accept_len;
    a.bonus = bonus;
    a.hit = hit;
    a.n_min = n_min;
    a.n_max = n_max;
    a.seed = rng.seed;
    a.round = rng.round;
    a.tokens = fallback_tokens;
    a.next_draft = next_draft;
    a.match_n = match_n;
    a.match_end = match_end;
    a.dev_err = dev_err;
    hipError_t e = ssd::launch_ngram(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "ssd_ngram_fallback");
    return SSD_OK;
}

ssd_status ssd_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0) return SSD_ERR_ARG;
    hipError_t e = ssd::launch_stream_read(buf, (int64_t)(bytes / 16), sink, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "ssd_stream_read");
    return SSD_OK;
}

// The fused round; round_dev (nullable) replaces rng.round by a counter the kernels read
// from device memory when they run.
// Argument checks of the fused round (everything but the workspace); O receives the
// fan-out offsets.
static ssd_status round_check(const ssd_shape* s, const void* p_logits, const void* q_logits, const int32_t* draft,
                              const int32_t* F_host, int32_t Bf, float C, int32_t fallback, const ssd_round_out* out,
                              int* O) {
    ssd_status st = check_shape(s);
    if (st != SSD_OK) return st;
    if ((st = check_fanout(s, F_host, Bf, O)) != SSD_OK) return st;
    if (!p_logits || !q_logits || !draft || !out || !(C > 0.f) || !(C <= 1.f)) return SSD_ERR_ARG;
    if (fallback != SSD_FALLBACK_NONE && fallback != SSD_FALLBACK_UNIFORM) return SSD_ERR_ARG;
    if ((Bf > 0 && !out->cache_ids) || !out->accept_len || !out->bonus || !out->hit || !out->slot ||
        !out->fallback_tokens)
        return SSD_ERR_ARG;
    if (out->next_draft && Bf > 0 && !out->cache_values) return SSD_ERR_ARG;
    return SSD_OK;
}

static ssd_status round_impl(const ssd_shape* s, const void* p_logits, const void* q_logits, const int32_t* draft,
                             const int32_t* F_host, int32_t Bf, float C, ssd_rng rng, const uint64_t* round_dev,
                             int32_t fallback, const ssd_round_out* out, const ssd_round_events* ev, void* ws,
                             size_t ws_bytes, void* stream) {
    int O[SSD_MAX_K + 2];
    ssd_status st = round_check(s, p_logits, q_logits, draft, F_host, Bf, C, fallback, out, O);
    if (st != SSD_OK) return st;
    Layout L;
    if ((st = check_ws(s, Bf, ws, ws_bytes, &L)) != SSD_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    const int K1 = s->K + 1, R = s->B * K1;
    const int greedy = s->T == 0.f;
    double* dstats = at<double>(ws, L.stats);
    float* fstats = reinterpret_cast<float*>(dstats + 4 * R);
    int32_t* istats = reinterpret_cast<int32_t*>(fstats + 2 * R);
    ssd::Pass1Args a{};
    a.logits[0] = (const char*)p_logits;
    a.logits[1] = (const char*)q_logits;
    a.nmodel = 2;
    a.topf_model = 1;
    a.B = s->B;
    a.K1 = K1;
    a.V = s->V;
    a.ld_bytes = ld_bytes(s);
    a.c = temp_scale(s->T);
    a.greedy = greedy;
    a.want_arg = greedy || out->p_argmax || out->q_argmax;
    fill_fo(a, F_host, O, K1);
    set_ws(a, ws, L);
    a.draft = draft;
    a.probe = at<float>(ws, L.probe);

    ssd::SeqFinal f{};
    f.part = a.part;
    f.cand = a.cand;
    f.p_logits = a.logits[0];
    f.q_logits = a.logits[1];
    f.B = s->B;
    f.K = s->K;
    f.V = s->V;
    f.nt = a.nt;
    f.cap = a.cap;
    f.ld_bytes = a.ld_bytes;
    f.c = a.c;
    f.greedy = greedy;
    for (int i = 0; i <= ssd::kMaxKc; ++i) f.F[i] = a.F[i];
    for (int i = 0; i <= ssd::kMaxKc + 1; ++i) f.O[i] = a.O[i];
    f.draft = draft;
    f.probe = a.probe;
    f.C = C;
    f.seed = rng.seed;
    f.round = rng.round;
    f.round_ptr = round_dev;
    f.fallback = fallback;
    f.Bf = Bf;
    f.p_max = out->p_max ? out->p_max : fstats + 0 * R;
    f.p_sum = out->p_sum ? out->p_sum : dstats + 0 * R;
    f.q_max = out->q_max ? out->q_max : fstats + 1 * R;
    f.q_sum = out->q_sum ? out->q_sum : dstats + 1 * R;
    f.p_arg = out->p_argmax ? out->p_argmax : istats;
    f.q_arg = out->q_argmax;
    f.cache_ids = out->cache_ids;
    f.cache_mass = out->cache_mass ? out->cache_mass : dstats + 2 * R;
    f.Z = out->Z ? out->Z : dstats + 3 * R;
    f.accept_len = out->accept_len;
    f.accept_prob = out->accept_prob;
    f.bonus = out->bonus;
    f.resid_mass = out->resid_mass;
    f.hit = out->hit;
    f.slot = out->slot;
    f.fallback_tokens = out->fallback_tokens;
    f.dev_err = out->dev_err;
    f.vflag = at<int32_t>(ws, L.vflag);
    f.cache_values = out->cache_values;
    f.next_draft = out->next_draft;
    f.law = at<ssd::LawParams>(ws, L.law);

    const bool vec = vec_ok(s, p_logits) && vec_ok(s, q_logits);
    hipError_t e;
    if (ev && ev->pass1_start && (e = hipEventRecord((hipEvent_t)ev->pass1_start, hs)) != hipSuccess)
        return fail_hip(e, "ssd_round event");
    e = ssd::launch_pass1(s->dtype, vec, a, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_round pass 1");
    if (ev && ev->pass1_stop && (e = hipEventRecord((hipEvent_t)ev->pass1_stop, hs)) != hipSuccess)
        return fail_hip(e, "ssd_round event");
    e = ssd::launch_finalize_pos(s->dtype, f, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_round finalise");
    if (greedy) {
        e = ssd::launch_finish_greedy(f, hs);
        if (e != hipSuccess) return fail_hip(e, "ssd_round greedy bonus");
        return SSD_OK;
    }

    ssd::Pass2Args b{};
    b.p_logits = (const char*)p_logits;
    b.q_logits = (const char*)q_logits;
    b.B = s->B;
    b.K = s->K;
    b.V = s->V;
    b.ld_bytes = a.ld_bytes;
    b.c = a.c;
    b.C = C;
    b.mode = 0;
    b.nt = L.nt2;
    fill_fo(b, F_host, O, K1);
    b.Bf = Bf;
    b.p_max = f.p_max;
    b.p_sum = f.p_sum;
    b.q_max = f.q_max;
    b.q_sum = f.q_sum;
    b.Z = f.Z;
    b.cache_ids = f.cache_ids;
    b.vflag = f.vflag;
    b.accept_len_out = f.accept_len;
    b.seed = rng.seed;
    b.round = rng.round;
    b.round_ptr = round_dev;
    b.seg = at<double2>(ws, L.seg);
    b.out_tok = out->bonus;
    b.resid_mass = out->resid_mass;
    b.dev_err = out->dev_err;
    b.do_lookup = 1;
    b.cache_values = out->cache_values;
    b.next_draft = out->next_draft;
    b.fallback = fallback;
    b.hit = out->hit;
    b.slot = out->slot;
    b.fallback_tokens = out->fallback_tokens;
    b.law = f.law;
    if (ev && ev->pass2_start && (e = hipEventRecord((hipEvent_t)ev->pass2_start, hs)) != hipSuccess)
        return fail_hip(e, "ssd_round event");
    e = ssd::launch_pass2(s->dtype, vec, b, s->B, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_round pass 2");
    if (ev && ev->pass2_stop && (e = hipEventRecord((hipEvent_t)ev->pass2_stop, hs)) != hipSuccess)
        return fail_hip(e, "ssd_round event");
    e = ssd::launch_finalize_bonus(s->dtype, vec, b, s->B, hs);
    if (e != hipSuccess) return fail_hip(e, "ssd_round bonus");
    return SSD_OK;
}

ssd_status ssd_round(const ssd_shape* s, const void* p_logits, const void* q_logits, const int32_t* draft,
                     const int32_t* F_host, int32_t Bf, float C, ssd_rng rng, int32_t fallback,
                     const ssd_round_out* out, const ssd_round_events* ev, void* ws, size_t ws_bytes, void* stream) {
    return round_impl(s, p_logits, q_logits, draft, F_host, Bf, C, rng, nullptr, fallback, out, ev, ws, ws_bytes,
                      stream);
}

ssd_status ssd_round_noalloc(const ssd_shape* s, const void* p_logits, const void* q_logits, const int32_t* draft,
                             const int32_t* F_host, int32_t Bf, float C, ssd_rng rng, int32_t fallback,
                             const ssd_round_out* out, const ssd_round_events* ev, void* stream) {
    int O[SSD_MAX_K + 2];
    ssd_status st = round_check(s, p_logits, q_logits, draft, F_host, Bf, C, fallback, out, O);
    if (st != SSD_OK) return st;
    Layout L;
    layout_for(s, Bf, &L);
    if (L.total > SSD_NOALLOC_SCRATCH_BYTES) {
        snprintf(g_last_error, sizeof(g_last_error),
                 "ssd_round_noalloc: the round needs %zu bytes of scratch, the static array holds %zu", L.total,
                 (size_t)SSD_NOALLOC_SCRATCH_BYTES);
        return SSD_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    if ((st = scratch_for((hipStream_t)stream, &ws)) != SSD_OK) return st;
    return round_impl(s, p_logits, q_logits, draft, F_host, Bf, C, rng, nullptr, fallback, out, ev, ws,
                      SSD_NOALLOC_SCRATCH_BYTES, stream);
}

ssd_status ssd_round_devrng(const ssd_shape* s, const void* p_logits, const void* q_logits, const int32_t* draft,
                            const int32_t* F_host, int32_t Bf, float C, uint64_t seed, const uint64_t* round_dev,
                            int32_t fallback, const ssd_round_out* out, const ssd_round_events* ev, void* ws,
                            size_t ws_bytes, void* stream) {
    if (!round_dev) return SSD_ERR_ARG;
    const ssd_rng rng{seed, 0};
    return round_impl(s, p_logits, q_logits, draft, F_host, Bf, C, rng, round_dev, fallback, out, ev, ws, ws_bytes,
                      stream);
}

}  // extern "C"
