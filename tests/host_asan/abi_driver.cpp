// Host-side check of the C ABI under AddressSanitizer (host code only: the
// library's *_api.cpp sources and this driver are built with the sanitizer,
// the GPU kernels are not). Every call of include/onela.h is made, on valid
// and invalid arguments, with host output buffers of exactly the documented
// size, so that a host-side overrun, use after free or double free in the
// library is reported by the sanitizer. Exit status 0 and a final "0 failed"
// line mean every status matched its documented value.
#include "onela.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

static int g_checks = 0, g_failed = 0;

#define CHECK(expr)                                                               \
    do {                                                                          \
        ++g_checks;                                                               \
        if (!(expr)) {                                                            \
            ++g_failed;                                                           \
            std::fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #expr); \
        }                                                                         \
    } while (0)

namespace {

uint16_t bf16_bits(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    u += 0x7FFF + ((u >> 16) & 1);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T>
T* to_device(const std::vector<T>& h) {
    T* d = nullptr;
    if (hipMalloc(&d, h.size() * sizeof(T)) != hipSuccess) return nullptr;
    if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
    return d;
}

struct StepInputs {
    uint16_t *q = nullptr, *k = nullptr, *v = nullptr;
    float *alpha = nullptr, *beta = nullptr, *o = nullptr, *delta = nullptr;
    int32_t* parents = nullptr;
};

StepInputs make_inputs(std::mt19937& rng, int n, int W, int H, int d) {
    std::normal_distribution<float> nd(0.f, 1.f);
    std::uniform_real_distribution<float> ud(0.05f, 0.95f);
    std::uniform_int_distribution<int> pd(0, W - 1);
    const size_t rows = static_cast<size_t>(n) * W * H;
    std::vector<uint16_t> q(rows * d), k(rows * d), v(rows * d);
    for (size_t r = 0; r < rows; ++r) {
        float nq = 0.f, nk = 0.f, xq[128], xk[128];
        for (int e = 0; e < d; ++e) {
            xq[e] = nd(rng);
            xk[e] = nd(rng);
            nq += xq[e] * xq[e];
            nk += xk[e] * xk[e];
        }
        for (int e = 0; e < d; ++e) {
            q[r * d + e] = bf16_bits(xq[e] / std::sqrt(nq));
            k[r * d + e] = bf16_bits(xk[e] / std::sqrt(nk));
            v[r * d + e] = bf16_bits(nd(rng));
        }
    }
    std::vector<float> a(rows), b(rows);
    for (size_t r = 0; r < rows; ++r) {
        a[r] = ud(rng);
        b[r] = ud(rng);
    }
    std::vector<int32_t> p(static_cast<size_t>(n) * W);
    for (auto& x : p) x = pd(rng);
    StepInputs in;
    in.q = to_device(q);
    in.k = to_device(k);
    in.v = to_device(v);
    in.alpha = to_device(a);
    in.beta = to_device(b);
    in.parents = to_device(p);
    std::vector<float> zeros(rows * d, 0.f);
    in.o = to_device(zeros);
    in.delta = to_device(zeros);
    return in;
}

void free_inputs(StepInputs& in) {
    for (void* p : {(void*)in.q, (void*)in.k, (void*)in.v, (void*)in.alpha, (void*)in.beta, (void*)in.o,
                    (void*)in.delta, (void*)in.parents})
        if (p) (void)hipFree(p);
    in = StepInputs{};
}

}  // namespace

int main() {
    const int R = 3, H = 2, D = 32, W = 40, T = 4;
    std::mt19937 rng(20261203);

    // ---- create: invalid configurations, then a valid one --------------------
    onela_ctx* ctx = nullptr;
    onela_config bad{0, H, D, D, W, T};
    CHECK(onela_create(&bad, nullptr, &ctx) == ONELA_E_INVALID_ARG && ctx == nullptr);
    bad = onela_config{R, H, 48, 48, W, T};
    CHECK(onela_create(&bad, nullptr, &ctx) == ONELA_E_UNSUPPORTED);
    bad = onela_config{R, H, D, D, W, ONELA_MAX_STEPS + 1};
    CHECK(onela_create(&bad, nullptr, &ctx) == ONELA_E_UNSUPPORTED);
    CHECK(onela_create(nullptr, nullptr, &ctx) == ONELA_E_INVALID_ARG);
    const onela_config cfg{R, H, D, D, W, T};
    CHECK(onela_create(&cfg, nullptr, nullptr) == ONELA_E_INVALID_ARG);
    CHECK(onela_create(&cfg, nullptr, &ctx) == ONELA_OK && ctx != nullptr);
    if (!ctx) {
        std::printf("host-asan driver: %d checks, %d failed (no context)\n", g_checks, g_failed);
        return 1;
    }

    // ---- S0 and requests -------------------------------------------------------
    std::vector<float> s0h(static_cast<size_t>(H) * D * D);
    std::normal_distribution<float> nd(0.f, 0.1f);
    for (auto& x : s0h) x = nd(rng);
    float* S0 = to_device(s0h);
    CHECK(onela_init_request(ctx, 0, S0) == ONELA_OK);
    CHECK(onela_init_request(ctx, 1, S0) == ONELA_OK);
    CHECK(onela_init_request(ctx, R, S0) == ONELA_E_INVALID_ARG);
    CHECK(onela_init_request(ctx, 0, nullptr) == ONELA_E_INVALID_ARG);

    StepInputs in = make_inputs(rng, 2, W, H, D);
    const int32_t both[2] = {0, 1}, dup[2] = {1, 1}, out_of_range[2] = {0, R}, fresh[1] = {2};
    CHECK(onela_step(ctx, 2, dup, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) == ONELA_E_INVALID_ARG);
    CHECK(onela_step(ctx, 2, out_of_range, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) ==
          ONELA_E_INVALID_ARG);
    CHECK(onela_step(ctx, 0, both, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) == ONELA_E_INVALID_ARG);
    CHECK(onela_step(ctx, 1, fresh, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) == ONELA_E_BAD_STATE);
    CHECK(onela_step(ctx, 2, both, nullptr, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) ==
          ONELA_E_INVALID_ARG);

    // ---- an episode: launch-shape knobs, then every step -----------------------
    CHECK(onela_set_beams_per_block(ctx, 100) == ONELA_E_INVALID_ARG);
    CHECK(onela_set_beam_order(ctx, 2) == ONELA_E_INVALID_ARG);
    CHECK(onela_set_beam_order(nullptr, 0) == ONELA_E_INVALID_ARG);
    CHECK(onela_set_beams_per_block(ctx, 64) == ONELA_OK);
    for (int t = 0; t < T; ++t) {
        CHECK(onela_set_beam_order(ctx, t % 3 - 1) == ONELA_OK);
        const int32_t* par = t ? in.parents : nullptr;
        CHECK(onela_step(ctx, 2, both, in.q, in.k, in.v, in.alpha, in.beta, par, in.o, in.delta) == ONELA_OK);
    }
    CHECK(onela_step(ctx, 2, both, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) ==
          ONELA_E_CAPACITY);
    CHECK(onela_sync(ctx) == ONELA_OK);

    // ---- inspection into buffers of exactly the documented size ----------------
    int32_t t_done = -1;
    CHECK(onela_get_step(ctx, 0, &t_done) == ONELA_OK && t_done == T);
    CHECK(onela_get_step(ctx, R, &t_done) == ONELA_E_INVALID_ARG);
    std::vector<int32_t> anc(static_cast<size_t>(W) * T);
    CHECK(onela_get_ancestry(ctx, 1, anc.data()) == ONELA_OK);
    bool anc_ok = true;
    for (int b = 0; b < W; ++b)
        for (int j = 0; j < T; ++j) {
            const int32_t id = anc[static_cast<size_t>(b) * T + j];
            anc_ok &= j < T - 1 ? (id >= j * W && id < (j + 1) * W) : id == -1;
        }
    CHECK(anc_ok);
    const int n_rec = T * W;
    std::vector<float> ra(n_rec), rd(static_cast<size_t>(n_rec) * D);
    std::vector<uint16_t> rk(static_cast<size_t>(n_rec) * D);
    CHECK(onela_get_records(ctx, 1, H - 1, n_rec, ra.data(), rd.data(), rk.data()) == ONELA_OK);
    CHECK(onela_get_records(ctx, 1, H - 1, n_rec, nullptr, rd.data(), nullptr) == ONELA_OK);
    CHECK(onela_get_records(ctx, 1, 0, n_rec - W + 3, ra.data(), rd.data(), rk.data()) == ONELA_OK);   // ends inside a step
    CHECK(onela_get_records(ctx, 1, H, n_rec, ra.data(), nullptr, nullptr) == ONELA_E_INVALID_ARG);
    CHECK(onela_get_records(ctx, 1, 0, n_rec + 1, ra.data(), nullptr, nullptr) == ONELA_E_INVALID_ARG);
    uint64_t s0b = 0, recb = 0, idxb = 0;
    CHECK(onela_get_memory(ctx, &s0b, &recb, &idxb) == ONELA_OK && s0b > 0 && recb > 0 && idxb > 0);

    // ---- a bad parent poisons the request until it restarts --------------------
    CHECK(onela_reset(ctx, 0) == ONELA_OK);
    CHECK(onela_reset(ctx, R) == ONELA_E_INVALID_ARG);
    const int32_t one[1] = {0};
    CHECK(onela_step(ctx, 1, one, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) == ONELA_OK);
    std::vector<int32_t> badp(W, 0);
    badp[7] = W;
    int32_t* dbad = to_device(badp);
    CHECK(onela_step(ctx, 1, one, in.q, in.k, in.v, in.alpha, in.beta, dbad, in.o, nullptr) == ONELA_OK);
    CHECK(onela_sync(ctx) == ONELA_E_PARENT_RANGE);
    CHECK(onela_step(ctx, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) ==
          ONELA_E_BAD_STATE);
    CHECK(onela_init_request(ctx, 0, S0) == ONELA_OK);
    CHECK(onela_sync(ctx) == ONELA_OK);

    // ---- input-side fusion -----------------------------------------------------
    std::vector<float> alog(H, 0.5f), dtb(H, -3.f);
    float* dA = to_device(alog);
    float* dD = to_device(dtb);
    onela_gate_params gates{dA, dD, 1e-6f};
    CHECK(onela_step_raw(ctx, 1, one, in.q, in.k, in.v, in.alpha, in.beta, &gates, nullptr,
                         reinterpret_cast<uint16_t*>(in.o), nullptr) == ONELA_OK);
    onela_gate_params neg{dA, dD, -1.f};
    CHECK(onela_step_raw(ctx, 1, one, in.q, in.k, in.v, in.alpha, in.beta, &neg, in.parents,
                         reinterpret_cast<uint16_t*>(in.o), nullptr) == ONELA_E_INVALID_ARG);
    CHECK(onela_sync(ctx) == ONELA_OK);

    // ---- prompts: into the context's planes, and into float32 states ----------
    const int L = 20;
    StepInputs pr = make_inputs(rng, 1, L, H, D);   // [1][L][H][d] prompt tokens
    CHECK(onela_init_requests_from_prompts(ctx, 1, one, L, pr.k, pr.v, pr.alpha, pr.beta) == ONELA_OK);
    CHECK(onela_init_requests_from_prompts(ctx, 2, dup, L, pr.k, pr.v, pr.alpha, pr.beta) == ONELA_E_INVALID_ARG);
    float* states = nullptr;
    CHECK(hipMalloc(&states, sizeof(float) * H * D * D) == hipSuccess);
    CHECK(onela_prefill(1, H, D, D, L, pr.k, pr.v, pr.alpha, pr.beta, nullptr, states, nullptr) == ONELA_OK);
    CHECK(onela_prefill(1, H, D, D, L, pr.k, pr.v, pr.alpha, pr.beta, states, states, nullptr) == ONELA_OK);
    CHECK(onela_prefill(1, H, 48, 48, L, pr.k, pr.v, pr.alpha, pr.beta, nullptr, states, nullptr) ==
          ONELA_E_UNSUPPORTED);
    CHECK(hipDeviceSynchronize() == hipSuccess);

    // ---- a layer sharing the index, and graph mode -----------------------------
    onela_ctx* sharer = nullptr;
    CHECK(onela_create_sharing_index(&cfg, nullptr, ctx, &sharer) == ONELA_OK && sharer != nullptr);
    if (sharer) {
        CHECK(onela_init_request(sharer, 0, S0) == ONELA_OK);
        CHECK(onela_reset(ctx, 0) == ONELA_OK);
        CHECK(onela_step(ctx, 1, one, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) == ONELA_OK);
        CHECK(onela_step(sharer, 1, one, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) == ONELA_OK);
        // the sharer's step 2 reads the rows of the owner's step 1 and the beam
        // order of the owner's step 2; its step 3 would need the owner's step 3
        CHECK(onela_step(sharer, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) ==
              ONELA_E_BAD_STATE);
        CHECK(onela_step(ctx, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) == ONELA_OK);
        CHECK(onela_step(sharer, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) == ONELA_OK);
        CHECK(onela_step(sharer, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) ==
              ONELA_E_BAD_STATE);
        CHECK(onela_destroy(ctx) == ONELA_E_BAD_STATE);   // still shared
        CHECK(onela_set_graph_mode(ctx, 1) == ONELA_OK);
        CHECK(onela_set_graph_mode(sharer, 1) == ONELA_OK);
        CHECK(onela_step(ctx, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) == ONELA_OK);
        CHECK(onela_step(sharer, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) ==
              ONELA_OK);
        CHECK(onela_sync(ctx) == ONELA_OK && onela_sync(sharer) == ONELA_OK);
        CHECK(onela_get_step(ctx, 0, &t_done) == ONELA_OK && t_done == 3);
        CHECK(onela_get_step(sharer, 0, &t_done) == ONELA_OK && t_done == 3);
        CHECK(onela_set_graph_mode(sharer, 0) == ONELA_OK);
        CHECK(onela_set_graph_mode(ctx, 0) == ONELA_OK);
        CHECK(onela_destroy(sharer) == ONELA_OK);
    }

    // ---- status text -----------------------------------------------------------
    for (int s = 1; s >= -8; --s) CHECK(onela_status_string(s) != nullptr);
    CHECK(onela_last_error(ctx) != nullptr);
    CHECK(onela_destroy(ctx) == ONELA_OK);
    CHECK(onela_destroy(nullptr) == ONELA_OK);

    // ---- the comparators -------------------------------------------------------
    onela_fs_ctx* fs = nullptr;
    CHECK(onela_fs_create(&cfg, nullptr, &fs) == ONELA_OK && fs != nullptr);
    if (fs) {
        CHECK(onela_fs_init_request(fs, 0, S0) == ONELA_OK);
        CHECK(onela_fs_step(fs, 1, one, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, in.delta) == ONELA_OK);
        CHECK(onela_fs_step(fs, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) == ONELA_OK);
        CHECK(onela_fs_step(fs, 1, fresh, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, nullptr) ==
              ONELA_E_BAD_STATE);
        CHECK(onela_fs_sync(fs) == ONELA_OK);
        uint64_t bytes = 0;
        CHECK(onela_fs_get_memory(fs, &bytes) == ONELA_OK && bytes > 0);
        CHECK(onela_fs_reset(fs, 0) == ONELA_OK);
        CHECK(onela_fs_destroy(fs) == ONELA_OK);
    }
    onela_rs_ctx* rs = nullptr;
    CHECK(onela_rs_create(&cfg, nullptr, &rs) == ONELA_OK && rs != nullptr);
    if (rs) {
        CHECK(onela_rs_init_request(rs, 0, S0) == ONELA_OK);
        CHECK(onela_rs_step(rs, 1, one, in.q, in.k, in.v, in.alpha, in.beta, nullptr, in.o, in.delta) == ONELA_OK);
        CHECK(onela_rs_step(rs, 1, one, in.q, in.k, in.v, in.alpha, in.beta, in.parents, in.o, nullptr) == ONELA_OK);
        CHECK(onela_rs_sync(rs) == ONELA_OK);
        uint64_t bytes = 0;
        CHECK(onela_rs_get_memory(rs, &bytes) == ONELA_OK && bytes > 0);
        CHECK(onela_rs_reset(rs, 0) == ONELA_OK);
        CHECK(onela_rs_destroy(rs) == ONELA_OK);
    }

    free_inputs(in);
    free_inputs(pr);
    for (void* p : {(void*)S0, (void*)dbad, (void*)dA, (void*)dD, (void*)states}) (void)hipFree(p);
    std::printf("host-asan driver: %d checks, %d failed\n", g_checks, g_failed);
    return g_failed == 0 ? 0 : 1;
}
