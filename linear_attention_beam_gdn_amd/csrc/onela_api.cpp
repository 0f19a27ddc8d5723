// Host runtime and C ABI of the OneLA GDN decode step (declared in onela.h).
//
// A context is one GDN layer: fixed-capacity, library-owned device buffers
// for the shared states, the append-only record store and the ancestry index,
// plus host-side step counters per request. onela_step validates on the host,
// then enqueues one step launch per group of up to kMaxReqPerLaunch requests.
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/onela.h"
#include "onela_internal.h"

struct onela_ctx {
    onela_config cfg;
    hipStream_t stream = nullptr;
    int device = 0;
    uint16_t* s0_planes = nullptr;
    float* rec_alpha = nullptr;
    float* rec_delta = nullptr;
    uint16_t* rec_k = nullptr;
    int32_t* anc = nullptr;
    int32_t* order = nullptr;
    int32_t* order_hist = nullptr;   // null when W > kOrderMax: records then sit at their beam index
    int32_t* err = nullptr;
    std::vector<int32_t> steps;      // steps done per request; -1 = never initialised
    std::vector<char> poisoned;      // a bad parent index was reported
    std::vector<int32_t> err_host;
    std::vector<int32_t> epoch;      // episode number per request; a device error word counts only
                                     // if it carries the current one, so reset needs no device work
    int32_t beams_per_block = 0;     // 0 = automatic
    int32_t beam_order = -1;         // -1 = automatic, 0 = beam-index order, 1 = ancestry order
    std::string last_error;
    uint64_t s0_bytes = 0, rec_bytes = 0, idx_bytes = 0;
    // Layers of one model share one ancestry index: the owner allocates and
    // writes it, every sharing context only reads it.
    onela_ctx* index_owner = nullptr;
    std::vector<onela_ctx*> sharers;
    std::vector<char> stale;         // the owner restarted the request; this context must too
    // Graph mode: the device holds each request's step and episode number, so
    // captured onela_step launches advance correctly on every replay.
    bool graph_mode = false;
    int32_t* dev_steps = nullptr;    // [R]
    int32_t* dev_epoch = nullptr;    // [R]
    int32_t* err_cap = nullptr;      // [R]
    int32_t* done = nullptr;         // [R] finished workgroups of the running launch (0 between launches)
    std::vector<char> capacity_hit;  // a graph-mode step ran past max_steps
};

namespace {

onela_status hip_fail(onela_ctx* ctx, hipError_t e, const char* what) {
    if (ctx) ctx->last_error = std::string(what) + ": " + hipGetErrorString(e);
    return ONELA_E_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_req(const onela_ctx* ctx, int32_t req) {
    return req >= 0 && req < ctx->cfg.max_requests;
}

// Request `req` starts a new episode on this context (init or reset); the
// device copies of its counters follow on the stream.
hipError_t restart(onela_ctx* ctx, int32_t req) {
    ctx->steps[req] = 0;
    ctx->poisoned[req] = 0;
    ctx->stale[req] = 0;
    ctx->capacity_hit[req] = 0;
    ctx->epoch[req] = ctx->epoch[req] == INT32_MAX ? 1 : ctx->epoch[req] + 1;
    for (onela_ctx* s : ctx->sharers)            // their copies of the episode no longer match the index
        if (s->steps[req] > 0) s->stale[req] = 1;
    if (!ctx->graph_mode) return hipSuccess;     // host-only outside graph mode
    return onela::launch_set_counters(ctx->dev_steps, ctx->dev_epoch, req, 0, ctx->epoch[req], ctx->stream);
}

// Copy the device error words to the host and poison every flagged request;
// in graph mode also take the device's step counters as the host's.
onela_status drain(onela_ctx* ctx) {
    const size_t bytes = sizeof(int32_t) * ctx->cfg.max_requests;
    hipError_t e = hipStreamSynchronize(ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamSynchronize");
    e = hipMemcpy(ctx->err_host.data(), ctx->err, bytes, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy(err)");
    for (int r = 0; r < ctx->cfg.max_requests; ++r)
        if (ctx->err_host[r] != 0 && ctx->err_host[r] == ctx->epoch[r]) ctx->poisoned[r] = 1;
    if (ctx->graph_mode) {
        e = hipMemcpy(ctx->err_host.data(), ctx->err_cap, bytes, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy(err_cap)");
        for (int r = 0; r < ctx->cfg.max_requests; ++r)
            if (ctx->err_host[r] != 0 && ctx->err_host[r] == ctx->epoch[r]) ctx->capacity_hit[r] = 1;
        std::vector<int32_t> dsteps(ctx->cfg.max_requests);
        e = hipMemcpy(dsteps.data(), ctx->dev_steps, bytes, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy(steps)");
        for (int r = 0; r < ctx->cfg.max_requests; ++r)
            if (ctx->steps[r] >= 0) ctx->steps[r] = dsteps[r];
    }
    return ONELA_OK;
}

struct LaunchShape {
    int beams_per_block;
    bool half_chunks;   // the general body takes chunks of kChunk / 2 beams
    bool order_beams;   // beams processed in ancestry order
};

bool order_beams(const onela_ctx* ctx, int n_pairs, int beams_per_block) {
    const int W = ctx->cfg.beam_width;
    const int splits = (W + beams_per_block - 1) / beams_per_block;
    return (long)n_pairs * W >= onela::kOrderMinBeams && splits <= onela::kOrderMaxSplits;
}

LaunchShape auto_launch_shape(const onela_ctx* ctx, int n_pairs) {
    // Two workgroups fit on each of the 256 CUs: aim for at least 512 of
    // them, while keeping as many beams as possible per workgroup (its S0
    // slice stays in registers across them). A launch that cannot reach 512
    // workgroups with kChunk-beam chunks (few requests and heads) splits its
    // beams at half that length instead, for twice the workgroups.
    const int W = ctx->cfg.beam_width;
    const int want = (512 + n_pairs - 1) / n_pairs;
    const int chunks = (W + onela::kChunk - 1) / onela::kChunk;
    const bool half = chunks < want && W > onela::kChunk / 2;
    const int len = half ? onela::kChunk / 2 : onela::kChunk;
    const int n = (W + len - 1) / len;
    const int splits = std::max(1, std::min(n, want));
    const int bpb = ((n + splits - 1) / splits) * len;
    return {bpb, half, order_beams(ctx, n_pairs, bpb)};
}

}  // namespace

extern "C" {

const char* onela_status_string(onela_status s) {
    switch (s) {
        case ONELA_OK: return "ok";
        case ONELA_E_INVALID_ARG: return "invalid argument";
        case ONELA_E_BAD_STATE: return "request not initialised or poisoned";
        case ONELA_E_CAPACITY: return "request has no step left (max_steps reached)";
        case ONELA_E_PARENT_RANGE: return "parent index outside [0, W)";
        case ONELA_E_HIP: return "HIP error";
        case ONELA_E_OOM: return "device allocation failed";
        case ONELA_E_UNSUPPORTED: return "unsupported shape";
        default: return "unknown status";
    }
}

const char* onela_last_error(const onela_ctx* ctx) { return ctx ? ctx->last_error.c_str() : ""; }

static onela_status create_ctx(const onela_config* cfg, void* hip_stream, onela_ctx* owner, onela_ctx** out) {
    if (!out) return ONELA_E_INVALID_ARG;
    *out = nullptr;
    if (!cfg || cfg->max_requests < 1 || cfg->num_heads < 1 || cfg->beam_width < 1 || cfg->max_steps < 1 ||
        cfg->d_k < 1 || cfg->d_v < 1)
        return ONELA_E_INVALID_ARG;
    if (!onela::step_supported(cfg->d_k, cfg->d_v) || cfg->max_steps > ONELA_MAX_STEPS)
        return ONELA_E_UNSUPPORTED;
    // The kernels address one request's inputs and one (request, head)'s
    // records with 32-bit element offsets.
    const int64_t dmax = std::max(cfg->d_k, cfg->d_v);
    if ((int64_t)cfg->beam_width * cfg->num_heads * dmax >= INT32_MAX ||
        (int64_t)cfg->max_steps * cfg->beam_width * dmax >= INT32_MAX)
        return ONELA_E_UNSUPPORTED;

    onela_ctx* ctx = new onela_ctx();
    ctx->cfg = *cfg;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    (void)hipGetDevice(&ctx->device);
    const uint64_t R = cfg->max_requests, H = cfg->num_heads, W = cfg->beam_width, T = cfg->max_steps;
    const uint64_t dk = cfg->d_k, dv = cfg->d_v;
    const uint64_t nrec = R * H * T * W;
    ctx->s0_bytes = R * H * 2 * dv * dk * 2;
    ctx->rec_bytes = nrec * (4 + 4 * dv + 2 * dk);
    const bool track = W <= (uint64_t)onela::kOrderMax;
    ctx->idx_bytes = (owner ? 0 : 2 * R * W * T * 4 + 2 * R * W * 4 + (track ? R * T * W * 4 : 0)) +
                     5 * R * 4;   // + error words, counters

    bool ok = hipMalloc(&ctx->s0_planes, ctx->s0_bytes) == hipSuccess &&
              hipMalloc(&ctx->rec_alpha, nrec * 4) == hipSuccess &&
              hipMalloc(&ctx->rec_delta, nrec * 4 * dv) == hipSuccess &&
              hipMalloc(&ctx->rec_k, nrec * 2 * dk) == hipSuccess &&
              hipMalloc(&ctx->err, R * 4) == hipSuccess && hipMalloc(&ctx->dev_steps, R * 4) == hipSuccess &&
              hipMalloc(&ctx->dev_epoch, R * 4) == hipSuccess && hipMalloc(&ctx->err_cap, R * 4) == hipSuccess &&
              hipMalloc(&ctx->done, R * 4) == hipSuccess;
    if (ok && !owner)
        ok = hipMalloc(&ctx->anc, 2 * R * W * T * 4) == hipSuccess && hipMalloc(&ctx->order, 2 * R * W * 4) == hipSuccess &&
             (!track || hipMalloc(&ctx->order_hist, R * T * W * 4) == hipSuccess);
    if (!ok) {
        (void)hipGetLastError();
        onela_destroy(ctx);
        return ONELA_E_OOM;
    }
    if (hipMemsetAsync(ctx->err, 0, R * 4, ctx->stream) != hipSuccess ||
        hipMemsetAsync(ctx->err_cap, 0, R * 4, ctx->stream) != hipSuccess ||
        hipMemsetAsync(ctx->done, 0, R * 4, ctx->stream) != hipSuccess ||
        hipMemsetAsync(ctx->dev_steps, 0, R * 4, ctx->stream) != hipSuccess ||
        hipMemsetAsync(ctx->dev_epoch, 0, R * 4, ctx->stream) != hipSuccess ||
        (!owner && hipMemsetAsync(ctx->anc, 0xff, 2 * R * W * T * 4, ctx->stream) != hipSuccess) ||
        onela::prepare_step(cfg->d_k, cfg->d_v, cfg->max_steps, cfg->beam_width) != hipSuccess) {
        onela_destroy(ctx);
        return ONELA_E_HIP;
    }
    if (owner) {
        ctx->anc = owner->anc;
        ctx->order = owner->order;
        ctx->order_hist = owner->order_hist;
        ctx->index_owner = owner;
        owner->sharers.push_back(ctx);
    }
    ctx->stale.assign(R, 0);
    ctx->capacity_hit.assign(R, 0);
    ctx->steps.assign(R, -1);
    ctx->poisoned.assign(R, 0);
    ctx->err_host.assign(R, 0);
    ctx->epoch.assign(R, 0);
    *out = ctx;
    return ONELA_OK;
}

onela_status onela_create(const onela_config* cfg, void* hip_stream, onela_ctx** out) {
    return create_ctx(cfg, hip_stream, nullptr, out);
}

onela_status onela_create_sharing_index(const onela_config* cfg, void* hip_stream, onela_ctx* index_owner,
                                        onela_ctx** out) {
    if (!out) return ONELA_E_INVALID_ARG;
    *out = nullptr;
    if (!cfg || !index_owner || index_owner->index_owner) return ONELA_E_INVALID_ARG;
    const auto& oc = index_owner->cfg;
    if (cfg->max_requests != oc.max_requests || cfg->beam_width != oc.beam_width || cfg->max_steps != oc.max_steps)
        return ONELA_E_INVALID_ARG;
    return create_ctx(cfg, hip_stream, index_owner, out);
}

onela_status onela_destroy(onela_ctx* ctx) {
    if (!ctx) return ONELA_OK;
    if (!ctx->sharers.empty()) return ONELA_E_BAD_STATE;     // sharing contexts go first
    (void)hipStreamSynchronize(ctx->stream);
    (void)hipFree(ctx->s0_planes);
    (void)hipFree(ctx->rec_alpha);
    (void)hipFree(ctx->rec_delta);
    (void)hipFree(ctx->rec_k);
    if (ctx->index_owner) {
        auto& v = ctx->index_owner->sharers;
        v.erase(std::remove(v.begin(), v.end(), ctx), v.end());
    } else {
        (void)hipFree(ctx->anc);
        (void)hipFree(ctx->order);
        (void)hipFree(ctx->order_hist);
    }
    (void)hipFree(ctx->err);
    (void)hipFree(ctx->dev_steps);
    (void)hipFree(ctx->dev_epoch);
    (void)hipFree(ctx->err_cap);
    (void)hipFree(ctx->done);
    delete ctx;
    return ONELA_OK;
}

onela_status onela_init_request(onela_ctx* ctx, int32_t req, const float* S0) {
    if (!ctx || !S0 || !valid_req(ctx, req) || !aligned(S0, 16)) return ONELA_E_INVALID_ARG;
    const auto& c = ctx->cfg;
    uint16_t* planes = ctx->s0_planes + (size_t)req * c.num_heads * 2 * c.d_v * c.d_k;
    hipError_t e = onela::launch_init_s0(c.d_k, c.d_v, S0, planes, c.num_heads, ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "init_s0 launch");
    e = restart(ctx, req);
    return e == hipSuccess ? ONELA_OK : hip_fail(ctx, e, "counter launch");
}

onela_status onela_init_requests_from_prompts(onela_ctx* ctx, int32_t n_req, const int32_t* reqs, int32_t seq_len,
                                              const uint16_t* k, const uint16_t* v, const float* alpha,
                                              const float* beta) {
    if (!ctx || n_req < 1 || !reqs || seq_len < 0) return ONELA_E_INVALID_ARG;
    if (seq_len > 0 && (!k || !v || !alpha || !beta)) return ONELA_E_INVALID_ARG;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(alpha, 4) || !aligned(beta, 4)) return ONELA_E_INVALID_ARG;
    const auto& c = ctx->cfg;
    std::vector<char> seen(c.max_requests, 0);
    for (int i = 0; i < n_req; ++i) {
        if (!valid_req(ctx, reqs[i]) || seen[reqs[i]]) return ONELA_E_INVALID_ARG;
        seen[reqs[i]] = 1;
    }
    const size_t tok = (size_t)seq_len * c.num_heads;                 // rows of one request's prompt
    for (int i0 = 0; i0 < n_req; i0 += onela::kMaxReqPerLaunch) {
        const int n = std::min(onela::kMaxReqPerLaunch, n_req - i0);
        onela::PrefillParams p{};
        p.k = k ? k + i0 * tok * c.d_k : nullptr;
        p.v = v ? v + i0 * tok * c.d_v : nullptr;
        p.alpha = alpha ? alpha + i0 * tok : nullptr;
        p.beta = beta ? beta + i0 * tok : nullptr;
        p.s_init = nullptr;
        p.s_out = nullptr;
        p.planes = ctx->s0_planes;
        p.n_seq = n;
        p.H = c.num_heads;
        p.L = seq_len;
        for (int i = 0; i < n; ++i) p.slot[i] = reqs[i0 + i];
        hipError_t e = onela::launch_prefill(c.d_k, c.d_v, true, p, ctx->stream);
        if (e != hipSuccess) return hip_fail(ctx, e, "prefill launch");
    }
    for (int i = 0; i < n_req; ++i) {
        hipError_t e = restart(ctx, reqs[i]);
        if (e != hipSuccess) return hip_fail(ctx, e, "counter launch");
    }
    return ONELA_OK;
}

onela_status onela_reset(onela_ctx* ctx, int32_t req) {
    if (!ctx || !valid_req(ctx, req)) return ONELA_E_INVALID_ARG;
    if (ctx->steps[req] < 0) return ONELA_E_BAD_STATE;
    hipError_t e = restart(ctx, req);
    return e == hipSuccess ? ONELA_OK : hip_fail(ctx, e, "counter launch");
}

onela_status onela_set_graph_mode(onela_ctx* ctx, int32_t on) {
    if (!ctx || (on != 0 && on != 1)) return ONELA_E_INVALID_ARG;
    if ((bool)on == ctx->graph_mode) return ONELA_OK;
    onela_status st = drain(ctx);                 // (leaving graph mode: takes the device's step counters)
    if (st != ONELA_OK) return st;
    if (on) {
        const size_t bytes = sizeof(int32_t) * ctx->cfg.max_requests;
        std::vector<int32_t> zero(ctx->cfg.max_requests, 0), steps(ctx->steps);
        for (auto& x : steps) x = std::max(x, 0);
        hipError_t e = hipMemcpy(ctx->dev_steps, steps.data(), bytes, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(ctx->dev_epoch, ctx->epoch.data(), bytes, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(ctx->err_cap, zero.data(), bytes, hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy(counters)");
    }
    ctx->graph_mode = on;
    return ONELA_OK;
}

onela_status onela_set_beams_per_block(onela_ctx* ctx, int32_t beams) {
    if (!ctx || beams < 0 || beams % onela::kChunk != 0) return ONELA_E_INVALID_ARG;
    ctx->beams_per_block = beams;
    return ONELA_OK;
}

onela_status onela_set_beam_order(onela_ctx* ctx, int32_t mode) {
    if (!ctx || mode < -1 || mode > 1) return ONELA_E_INVALID_ARG;
    ctx->beam_order = mode;
    return ONELA_OK;
}

// One decode step for the listed requests. fused: q, k, alpha, beta are raw
// projections (gates non-null) and o goes to o16 as bf16; else o is float32.
static onela_status step_impl(onela_ctx* ctx, int32_t n_req, const int32_t* reqs, const uint16_t* q,
                              const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
                              const int32_t* parent_idx, float* o, uint16_t* o16, float* delta_out,
                              const onela_gate_params* gates) {
    const bool fused = gates != nullptr;
    if (!ctx || n_req < 1 || n_req > ctx->cfg.max_requests || !reqs || !q || !k || !v || !alpha || !beta ||
        (fused ? !o16 : !o))
        return ONELA_E_INVALID_ARG;
    if (fused && (!gates->A_log || !gates->dt_bias || !(gates->norm_eps >= 0.f))) return ONELA_E_INVALID_ARG;
    // vector loads and stores: 16 B for q, k, o, delta_out; 8 B for v and bf16 o; 4 B for the rest
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 8) || !aligned(o, 16) || !aligned(o16, 8) ||
        !aligned(delta_out, 16) || !aligned(alpha, 4) || !aligned(beta, 4) || !aligned(parent_idx, 4))
        return ONELA_E_INVALID_ARG;
    const auto& c = ctx->cfg;
    std::vector<char> seen(c.max_requests, 0);
    bool need_parents = false;
    for (int i = 0; i < n_req; ++i) {
        const int r = reqs[i];
        if (!valid_req(ctx, r) || seen[r]) return ONELA_E_INVALID_ARG;
        seen[r] = 1;
        if (ctx->steps[r] < 0 || ctx->poisoned[r] || ctx->stale[r]) return ONELA_E_BAD_STATE;
        if (ctx->graph_mode) {                    // the step index is known on the device only
            if (ctx->capacity_hit[r]) return ONELA_E_CAPACITY;
            need_parents = true;
            continue;
        }
        if (ctx->steps[r] >= c.max_steps) return ONELA_E_CAPACITY;
        if (ctx->steps[r] >= 1) need_parents = true;
        const int t = ctx->steps[r] + 1;
        // shared index: step t reads the rows the owner's step t-1 wrote, which
        // the owner's step t+1 overwrites, and the beam order of the owner's
        // step t (where its records go)
        if (ctx->index_owner && t >= 2 && ctx->index_owner->steps[r] != t) return ONELA_E_BAD_STATE;
        for (const onela_ctx* sh : ctx->sharers)
            if (t >= 2 && sh->steps[r] >= 1 && !sh->stale[r] && sh->steps[r] < t - 1) return ONELA_E_BAD_STATE;
    }
    if (need_parents && !parent_idx) return ONELA_E_INVALID_ARG;

    onela::StepParams p{};
    p.s0_planes = ctx->s0_planes;
    p.rec_alpha = ctx->rec_alpha;
    p.rec_delta = ctx->rec_delta;
    p.rec_k = ctx->rec_k;
    p.anc = ctx->anc;
    p.order = ctx->order;
    p.order_hist = ctx->order_hist;
    p.err = ctx->err;
    p.write_index = ctx->index_owner ? 0 : 1;
    p.dev_steps = ctx->graph_mode ? ctx->dev_steps : nullptr;
    p.dev_epoch = ctx->dev_epoch;
    p.err_cap = ctx->err_cap;
    p.done = ctx->done;
    if (fused) {
        p.A_log = gates->A_log;
        p.dt_bias = gates->dt_bias;
        p.norm_eps = gates->norm_eps;
    }
    p.H = c.num_heads;
    p.W = c.beam_width;
    p.T_max = c.max_steps;
    p.max_requests = c.max_requests;
    const size_t W = c.beam_width, H = c.num_heads;
    for (int i0 = 0; i0 < n_req; i0 += onela::kMaxReqPerLaunch) {
        const int n = std::min(onela::kMaxReqPerLaunch, n_req - i0);
        const size_t rows = (size_t)i0 * W;
        p.q = q + rows * H * c.d_k;
        p.k = k + rows * H * c.d_k;
        p.v = v + rows * H * c.d_v;
        p.alpha = alpha + rows * H;
        p.beta = beta + rows * H;
        p.parent = parent_idx ? parent_idx + rows : nullptr;
        p.o = o ? o + rows * H * c.d_v : nullptr;
        p.o_bf16 = o16 ? o16 + rows * H * c.d_v : nullptr;
        p.delta_out = delta_out ? delta_out + rows * H * c.d_v : nullptr;
        p.n_req = n;
        LaunchShape shape = auto_launch_shape(ctx, n * c.num_heads);
        if (ctx->beams_per_block)
            shape = {ctx->beams_per_block, false, order_beams(ctx, n * c.num_heads, ctx->beams_per_block)};
        if (ctx->beam_order >= 0) shape.order_beams = ctx->beam_order == 1;
        p.beams_per_block = shape.beams_per_block;
        p.order_beams = shape.order_beams ? 1 : 0;
        p.n_splits = (c.beam_width + p.beams_per_block - 1) / p.beams_per_block;
        for (int i = 0; i < n; ++i) {
            p.slot[i] = reqs[i0 + i];
            p.t[i] = ctx->steps[reqs[i0 + i]] + 1;
            p.epoch[i] = ctx->epoch[reqs[i0 + i]];
        }
        int n_first = 0;
        for (int i = 0; i < n; ++i) n_first += p.t[i] == 1;
        const int mode = ctx->graph_mode ? onela::kStepAny
                         : n_first == n  ? onela::kStepFirst
                         : n_first == 0  ? onela::kStepHist
                                         : onela::kStepAny;
        hipError_t e = onela::launch_step(c.d_k, c.d_v, fused, mode, shape.half_chunks, p, ctx->stream);
        if (e != hipSuccess) return hip_fail(ctx, e, "step launch");
        if (!ctx->graph_mode)                     // (graph mode: the launch advances the device counters)
            for (int i = 0; i < n; ++i) ctx->steps[reqs[i0 + i]] += 1;
    }
    return ONELA_OK;
}

onela_status onela_step(onela_ctx* ctx, int32_t n_req, const int32_t* reqs, const uint16_t* q,
                        const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
                        const int32_t* parent_idx, float* o, float* delta_out) {
    return step_impl(ctx, n_req, reqs, q, k, v, alpha, beta, parent_idx, o, nullptr, delta_out, nullptr);
}

onela_status onela_step_raw(onela_ctx* ctx, int32_t n_req, const int32_t* reqs, const uint16_t* q_raw,
                            const uint16_t* k_raw, const uint16_t* v, const float* a_raw, const float* b_raw,
                            const onela_gate_params* gates, const int32_t* parent_idx, uint16_t* o_bf16,
                            float* delta_out) {
    if (!gates) return ONELA_E_INVALID_ARG;
    return step_impl(ctx, n_req, reqs, q_raw, k_raw, v, a_raw, b_raw, parent_idx, nullptr, o_bf16, delta_out, gates);
}

onela_status onela_sync(onela_ctx* ctx) {
    if (!ctx) return ONELA_E_INVALID_ARG;
    onela_status s = drain(ctx);
    if (s != ONELA_OK) return s;
    for (int r = 0; r < ctx->cfg.max_requests; ++r)
        if (ctx->poisoned[r]) return ONELA_E_PARENT_RANGE;
    for (int r = 0; r < ctx->cfg.max_requests; ++r)
        if (ctx->capacity_hit[r]) return ONELA_E_CAPACITY;
    return ONELA_OK;
}

onela_status onela_get_step(onela_ctx* ctx, int32_t req, int32_t* t_done) {
    if (!ctx || !t_done || !valid_req(ctx, req)) return ONELA_E_INVALID_ARG;
    if (ctx->steps[req] < 0) return ONELA_E_BAD_STATE;
    onela_status s = drain(ctx);
    if (s != ONELA_OK) return s;
    *t_done = ctx->steps[req];
    return ctx->poisoned[req] ? ONELA_E_PARENT_RANGE : ONELA_OK;
}

// The beam at each processing position of the request's steps 1..n:
// ord[j*W + i] = beam written at record j*W + i (the identity when the
// kernels keep beam-index order, W > kOrderMax).
static hipError_t load_order(onela_ctx* ctx, int32_t req, int n, std::vector<int32_t>& ord) {
    const auto& c = ctx->cfg;
    const size_t W = c.beam_width;
    ord.resize((size_t)n * W);
    if (!ctx->order_hist) {
        for (size_t i = 0; i < ord.size(); ++i) ord[i] = (int32_t)(i % W);
        return hipSuccess;
    }
    if (n == 0) return hipSuccess;
    hipError_t e = hipMemcpy(ord.data(), ctx->order_hist + (size_t)req * c.max_steps * W, ord.size() * 4,
                             hipMemcpyDeviceToHost);
    for (int32_t& b : ord) b = (b < 0 || b >= (int32_t)W) ? 0 : b;   // (a valid order is a permutation)
    return e;
}

onela_status onela_get_ancestry(onela_ctx* ctx, int32_t req, int32_t* host_out) {
    if (!ctx || !host_out || !valid_req(ctx, req)) return ONELA_E_INVALID_ARG;
    if (ctx->steps[req] < 0) return ONELA_E_BAD_STATE;
    onela_status s = drain(ctx);
    if (s != ONELA_OK) return s;
    if (ctx->poisoned[req]) return ONELA_E_PARENT_RANGE;
    const auto& c = ctx->cfg;
    const size_t n = (size_t)c.beam_width * c.max_steps;
    const int t = ctx->steps[req];
    std::fill(host_out, host_out + n, -1);
    if (t >= 2) {
        std::vector<int32_t> buf(n), ord;
        const int32_t* src = ctx->anc + ((size_t)(t & 1) * c.max_requests + req) * n;
        hipError_t e = hipMemcpy(buf.data(), src, n * 4, hipMemcpyDeviceToHost);
        if (e == hipSuccess) e = load_order(ctx, req, t - 1, ord);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy(anc)");
        // stored ids name processing positions; reported ids name beams
        const int64_t W = c.beam_width;
        for (int b = 0; b < c.beam_width; ++b)
            for (int j = 0; j < t - 1; ++j) {
                const int32_t r = buf[(size_t)b * c.max_steps + j];
                host_out[(size_t)b * c.max_steps + j] =
                    (r >= 0 && r < (t - 1) * W) ? (int32_t)((r / W) * W + ord[r]) : r;
            }
    }
    return ONELA_OK;
}

onela_status onela_get_records(onela_ctx* ctx, int32_t req, int32_t head, int32_t n_rec, float* alpha,
                               float* delta, uint16_t* key) {
    if (!ctx || !valid_req(ctx, req) || head < 0 || head >= ctx->cfg.num_heads || n_rec < 0)
        return ONELA_E_INVALID_ARG;
    if (ctx->steps[req] < 0) return ONELA_E_BAD_STATE;
    const auto& c = ctx->cfg;
    onela_status s = drain(ctx);                  // (graph mode: refreshes the step counters)
    if (s != ONELA_OK) return s;
    if ((int64_t)n_rec > (int64_t)ctx->steps[req] * c.beam_width) return ONELA_E_INVALID_ARG;
    if (ctx->poisoned[req]) return ONELA_E_PARENT_RANGE;
    if (n_rec == 0) return ONELA_OK;
    // Stored record j*W + i belongs to the beam at position i of step j+1;
    // reported record (t-1)*W + b is beam b's.
    const size_t W = c.beam_width, NREC = (size_t)c.max_steps * W;
    const int n_steps = (int)((n_rec + W - 1) / W);
    const size_t n_st = (size_t)n_steps * W;      // stored records covering the reported ones
    std::vector<int32_t> ord;
    hipError_t e = load_order(ctx, req, n_steps, ord);
    std::vector<size_t> at(n_st);                 // stored index of reported record o
    for (size_t r = 0; r < n_st; ++r) at[(r / W) * W + ord[r]] = r;
    const size_t rec0 = ((size_t)req * c.num_heads + head) * NREC;
    if (e == hipSuccess && alpha) {
        std::vector<float> a(n_st);
        e = hipMemcpy(a.data(), ctx->rec_alpha + rec0, n_st * 4, hipMemcpyDeviceToHost);
        for (int o = 0; o < n_rec; ++o) alpha[o] = a[at[o]];
    }
    if (e == hipSuccess && delta) {
        std::vector<float> d(n_st * c.d_v);
        e = hipMemcpy(d.data(), ctx->rec_delta + rec0 * c.d_v, n_st * 4 * c.d_v, hipMemcpyDeviceToHost);
        for (int o = 0; o < n_rec; ++o)
            std::copy(&d[at[o] * c.d_v], &d[at[o] * c.d_v] + c.d_v, delta + (size_t)o * c.d_v);
    }
    if (e == hipSuccess && key) {
        std::vector<uint16_t> kb(n_st * c.d_k);
        e = hipMemcpy(kb.data(), ctx->rec_k + rec0 * c.d_k, n_st * 2 * c.d_k, hipMemcpyDeviceToHost);
        for (int o = 0; o < n_rec; ++o)
            std::copy(&kb[at[o] * c.d_k], &kb[at[o] * c.d_k] + c.d_k, key + (size_t)o * c.d_k);
    }
    if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy(records)");
    return ONELA_OK;
}

onela_status onela_get_memory(const onela_ctx* ctx, uint64_t* s0_bytes, uint64_t* record_bytes,
                              uint64_t* index_bytes) {
    if (!ctx) return ONELA_E_INVALID_ARG;
    if (s0_bytes) *s0_bytes = ctx->s0_bytes;
    if (record_bytes) *record_bytes = ctx->rec_bytes;
    if (index_bytes) *index_bytes = ctx->idx_bytes;
    return ONELA_OK;
}

}  // extern "C"
