// Host side of the replay comparator (declared in onela.h, "comparator").
//
// Same calling convention as onela_step. Persistent state: S0 per request and
// the append-only records (alpha, delta, k) of every beam, plus the parents
// given at every step; at each step every beam rebuilds its state from S0 and
// its own ancestral records.
#include <algorithm>
#include <vector>

#include "../../include/onela.h"
#include "onela_internal.h"

struct onela_rs_ctx {
    onela_config cfg;
    hipStream_t stream = nullptr;
    float* s0 = nullptr;
    float* rec_alpha = nullptr;
    float* rec_delta = nullptr;
    uint16_t* rec_k = nullptr;
    int32_t* par_hist = nullptr;
    int32_t* err = nullptr;
    std::vector<int32_t> steps, epoch, err_host;
    std::vector<char> poisoned;
    uint64_t state_bytes = 0;
};

namespace {

bool rs_valid_req(const onela_rs_ctx* c, int32_t r) { return r >= 0 && r < c->cfg.max_requests; }

bool rs_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

onela_status rs_drain(onela_rs_ctx* c) {
    if (hipStreamSynchronize(c->stream) != hipSuccess) return ONELA_E_HIP;
    if (hipMemcpy(c->err_host.data(), c->err, 4 * c->cfg.max_requests, hipMemcpyDeviceToHost) != hipSuccess)
        return ONELA_E_HIP;
    for (int r = 0; r < c->cfg.max_requests; ++r)
        if (c->err_host[r] != 0 && c->err_host[r] == c->epoch[r]) c->poisoned[r] = 1;
    return ONELA_OK;
}

void rs_restart(onela_rs_ctx* c, int32_t req) {
    c->steps[req] = 0;
    c->poisoned[req] = 0;
    c->epoch[req] = c->epoch[req] == INT32_MAX ? 1 : c->epoch[req] + 1;
}

}  // namespace

extern "C" {

onela_status onela_rs_create(const onela_config* cfg, void* hip_stream, onela_rs_ctx** out) {
    if (!out) return ONELA_E_INVALID_ARG;
    *out = nullptr;
    if (!cfg || cfg->max_requests < 1 || cfg->num_heads < 1 || cfg->beam_width < 1 || cfg->max_steps < 1 ||
        cfg->d_k < 1 || cfg->d_v < 1)
        return ONELA_E_INVALID_ARG;
    if (!onela::step_supported(cfg->d_k, cfg->d_v) || cfg->max_steps > ONELA_MAX_STEPS) return ONELA_E_UNSUPPORTED;
    if ((int64_t)cfg->beam_width * cfg->num_heads * std::max(cfg->d_k, cfg->d_v) >= INT32_MAX)
        return ONELA_E_UNSUPPORTED;
    onela_rs_ctx* c = new onela_rs_ctx();
    c->cfg = *cfg;
    c->stream = static_cast<hipStream_t>(hip_stream);
    const uint64_t R = cfg->max_requests, H = cfg->num_heads, W = cfg->beam_width, T = cfg->max_steps;
    const uint64_t dk = cfg->d_k, dv = cfg->d_v;
    const uint64_t nrec = R * H * T * W;
    const uint64_t s0_bytes = R * H * dv * dk * 4, rec_bytes = nrec * (4 + 4 * dv + 2 * dk);
    const uint64_t hist_bytes = R * T * W * 4;
    c->state_bytes = s0_bytes + rec_bytes + hist_bytes;
    if (hipMalloc(&c->s0, s0_bytes) != hipSuccess || hipMalloc(&c->rec_alpha, nrec * 4) != hipSuccess ||
        hipMalloc(&c->rec_delta, nrec * 4 * dv) != hipSuccess || hipMalloc(&c->rec_k, nrec * 2 * dk) != hipSuccess ||
        hipMalloc(&c->par_hist, hist_bytes) != hipSuccess || hipMalloc(&c->err, R * 4) != hipSuccess) {
        (void)hipGetLastError();
        onela_rs_destroy(c);
        return ONELA_E_OOM;
    }
    if (hipMemsetAsync(c->err, 0, R * 4, c->stream) != hipSuccess ||
        hipMemsetAsync(c->par_hist, 0, hist_bytes, c->stream) != hipSuccess) {
        onela_rs_destroy(c);
        return ONELA_E_HIP;
    }
    c->steps.assign(R, -1);
    c->epoch.assign(R, 0);
    c->err_host.assign(R, 0);
    c->poisoned.assign(R, 0);
    *out = c;
    return ONELA_OK;
}

onela_status onela_rs_destroy(onela_rs_ctx* c) {
    if (!c) return ONELA_OK;
    (void)hipStreamSynchronize(c->stream);
    (void)hipFree(c->s0);
    (void)hipFree(c->rec_alpha);
    (void)hipFree(c->rec_delta);
    (void)hipFree(c->rec_k);
    (void)hipFree(c->par_hist);
    (void)hipFree(c->err);
    delete c;
    return ONELA_OK;
}

onela_status onela_rs_init_request(onela_rs_ctx* c, int32_t req, const float* S0) {
    if (!c || !S0 || !rs_valid_req(c, req) || !rs_aligned(S0, 4)) return ONELA_E_INVALID_ARG;
    const size_t n = (size_t)c->cfg.num_heads * c->cfg.d_v * c->cfg.d_k;
    if (hipMemcpyAsync(c->s0 + (size_t)req * n, S0, n * 4, hipMemcpyDeviceToDevice, c->stream) != hipSuccess)
        return ONELA_E_HIP;
    rs_restart(c, req);
    return ONELA_OK;
}

onela_status onela_rs_reset(onela_rs_ctx* c, int32_t req) {
    if (!c || !rs_valid_req(c, req)) return ONELA_E_INVALID_ARG;
    if (c->steps[req] < 0) return ONELA_E_BAD_STATE;
    rs_restart(c, req);
    return ONELA_OK;
}

onela_status onela_rs_step(onela_rs_ctx* c, int32_t n_req, const int32_t* reqs, const uint16_t* q,
                           const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
                           const int32_t* parent_idx, float* o, float* delta_out) {
    if (!c || n_req < 1 || n_req > c->cfg.max_requests || !reqs || !q || !k || !v || !alpha || !beta || !o)
        return ONELA_E_INVALID_ARG;
    if (!rs_aligned(q, 16) || !rs_aligned(k, 16) || !rs_aligned(v, 2) || !rs_aligned(o, 4) ||
        !rs_aligned(delta_out, 4) || !rs_aligned(alpha, 4) || !rs_aligned(beta, 4) || !rs_aligned(parent_idx, 4))
        return ONELA_E_INVALID_ARG;
    const auto& cf = c->cfg;
    std::vector<char> seen(cf.max_requests, 0);
    bool need_parents = false;
    for (int i = 0; i < n_req; ++i) {
        const int r = reqs[i];
        if (!rs_valid_req(c, r) || seen[r]) return ONELA_E_INVALID_ARG;
        seen[r] = 1;
        if (c->steps[r] < 0 || c->poisoned[r]) return ONELA_E_BAD_STATE;
        if (c->steps[r] >= cf.max_steps) return ONELA_E_CAPACITY;
        if (c->steps[r] >= 1) need_parents = true;
    }
    if (need_parents && !parent_idx) return ONELA_E_INVALID_ARG;
    onela::ReplayParams p{};
    p.s0 = c->s0;
    p.rec_alpha = c->rec_alpha;
    p.rec_delta = c->rec_delta;
    p.rec_k = c->rec_k;
    p.par_hist = c->par_hist;
    p.err = c->err;
    p.H = cf.num_heads;
    p.W = cf.beam_width;
    p.T_max = cf.max_steps;
    p.max_requests = cf.max_requests;
    const size_t W = cf.beam_width, H = cf.num_heads;
    for (int i0 = 0; i0 < n_req; i0 += onela::kMaxReqPerLaunch) {
        const int n = std::min(onela::kMaxReqPerLaunch, n_req - i0);
        const size_t rows = (size_t)i0 * W;
        p.q = q + rows * H * cf.d_k;
        p.k = k + rows * H * cf.d_k;
        p.v = v + rows * H * cf.d_v;
        p.alpha = alpha + rows * H;
        p.beta = beta + rows * H;
        p.parent = parent_idx ? parent_idx + rows : nullptr;
        p.o = o + rows * H * cf.d_v;
        p.delta_out = delta_out ? delta_out + rows * H * cf.d_v : nullptr;
        p.n_req = n;
        for (int i = 0; i < n; ++i) {
            p.slot[i] = reqs[i0 + i];
            p.t[i] = c->steps[reqs[i0 + i]] + 1;
            p.epoch[i] = c->epoch[reqs[i0 + i]];
        }
        if (onela::launch_replay_step(cf.d_k, cf.d_v, p, c->stream) != hipSuccess) return ONELA_E_HIP;
        for (int i = 0; i < n; ++i) c->steps[reqs[i0 + i]] += 1;
    }
    return ONELA_OK;
}

onela_status onela_rs_sync(onela_rs_ctx* c) {
    if (!c) return ONELA_E_INVALID_ARG;
    onela_status s = rs_drain(c);
    if (s != ONELA_OK) return s;
    for (int r = 0; r < c->cfg.max_requests; ++r)
        if (c->poisoned[r]) return ONELA_E_PARENT_RANGE;
    return ONELA_OK;
}

onela_status onela_rs_get_memory(const onela_rs_ctx* c, uint64_t* state_bytes) {
    if (!c || !state_bytes) return ONELA_E_INVALID_ARG;
    *state_bytes = c->state_bytes;
    return ONELA_OK;
}

}  // extern "C"
