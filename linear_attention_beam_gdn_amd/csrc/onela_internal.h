// Internal interface between the C-ABI host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace onela {

// Requests one step launch carries in its kernel arguments; onela_step splits
// larger calls into several launches.
constexpr int kMaxReqPerLaunch = 64;
// Beams one workgroup stages at a time (one chunk of the beam loop); launches
// without ancestral records use chunks of half that size.
constexpr int kChunk = 64;
// Widest beam set that is processed in ancestry order (the order lives in LDS).
constexpr int kOrderMax = 1024;
// Launches with fewer (request, head) beam sets than this many beams in all
// keep the natural beam order: they are bound by the latency of each
// workgroup's dependent loads, which the ordering lengthens by one round, not
// by the record traffic it saves. So do launches that split a beam set over
// more than kOrderMaxSplits workgroups: each workgroup orders all W beams (a
// comparison rank up to 256 beams, a radix sort above) to process only its
// share of them.
constexpr long kOrderMinBeams = 32768;
constexpr int kOrderMaxSplits = 2;

struct StepParams {
    // caller inputs / outputs
    const uint16_t* q;       // bf16 [n_req*W][H][DK]
    const uint16_t* k;       // bf16 [n_req*W][H][DK]
    const uint16_t* v;       // bf16 [n_req*W][H][DV]
    const float* alpha;      // [n_req*W][H]
    const float* beta;       // [n_req*W][H]
    const int32_t* parent;   // [n_req][W] (unused for requests at t == 1)
    float* o;                // [n_req*W][H][DV]
    float* delta_out;        // optional, like o
    // library state
    const uint16_t* s0_planes;  // [max_requests][H][2][DV*DK] in MFMA fragment order
    // Records: record j*W + i is the one of step j+1 written by the beam at
    // position i of that step's processing order (the beam index itself when
    // W > kOrderMax).
    float* rec_alpha;           // [max_requests][H][T_max*W]
    float* rec_delta;           // [max_requests][H][T_max*W][DV]
    uint16_t* rec_k;            // [max_requests][H][T_max*W][DK]
    int32_t* anc;               // [2][max_requests][W][T_max] record ids (ping-pong by step parity)
    int32_t* order;             // [2][max_requests][W] beam at each position (ping-pong by step parity)
    int32_t* order_hist;        // [max_requests][T_max][W] the same for every step (W <= kOrderMax)
    int32_t* err;               // [max_requests]: epoch of the last step that saw a bad parent
    // Graph mode (non-null dev_steps): each request's step and episode number
    // come from device memory, so a captured launch stays valid on replay.
    int32_t* dev_steps;         // [max_requests] steps done; the launch's last workgroup of a request advances it
    const int32_t* dev_epoch;   // [max_requests] episode number
    int32_t* err_cap;           // [max_requests]: epoch of a step past max_steps (nothing written)
    int32_t* done;              // [max_requests] workgroups of the launch that finished (0 between launches)
    int32_t H, W, T_max, max_requests;
    // Input-side fusion (the fused kernel variant): q, k, alpha, beta above are
    // raw projections; o_bf16 receives o instead of o.
    const float* A_log;         // [H]
    const float* dt_bias;       // [H]
    float norm_eps;
    uint16_t* o_bf16;           // [n_req*W][H][DV] bf16
    int32_t write_index;        // 1: this launch writes the next step's ancestry rows and order
    int32_t order_beams;        // 1: beams are processed in ancestry order (W <= kOrderMax only)
    int32_t beams_per_block;    // multiple of the chunk length, or >= W
    int32_t n_splits;           // ceil(W / beams_per_block)
    int32_t n_req;
    int32_t slot[kMaxReqPerLaunch];  // request id of call-local request i
    int32_t t[kMaxReqPerLaunch];     // step this launch performs for it (1-based)
    int32_t epoch[kMaxReqPerLaunch]; // its episode number (> 0), written to err on a bad parent
};

// The full-state comparator (every beam keeps its own d_v x d_k state).
struct FullStateParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* alpha;
    const float* beta;
    const int32_t* parent;
    float* o;
    float* delta_out;
    const float* s0;            // [max_requests][H][DV*DK] float32
    float* state;               // [2][max_requests][H][W][DV*DK] float32 (ping-pong by step parity)
    int32_t* err;               // [max_requests]
    int32_t H, W, max_requests;
    int32_t n_req;
    int32_t slot[kMaxReqPerLaunch];
    int32_t t[kMaxReqPerLaunch];
    int32_t epoch[kMaxReqPerLaunch];
};

// Replay comparator: every beam rebuilds its state from S0 and its own
// ancestral records at every step (no per-beam state is kept, nothing shared).
struct ReplayParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* alpha;
    const float* beta;
    const int32_t* parent;      // this step's parents [n_req][W] (null at t = 1)
    float* o;
    float* delta_out;
    const float* s0;            // [max_requests][H][DV*DK] float32
    float* rec_alpha;           // [max_requests][H][T_max*W]
    float* rec_delta;           // [max_requests][H][T_max*W][DV]
    uint16_t* rec_k;            // [max_requests][H][T_max*W][DK] bf16
    int32_t* par_hist;          // [max_requests][T_max][W]: row s = parents given at step s+1 (s >= 1)
    int32_t* err;               // [max_requests]
    int32_t H, W, T_max, max_requests;
    int32_t n_req;
    int32_t slot[kMaxReqPerLaunch];
    int32_t t[kMaxReqPerLaunch];
    int32_t epoch[kMaxReqPerLaunch];
};

// The prefill: one workgroup per (sequence, head) folds a prompt into a state.
struct PrefillParams {
    const uint16_t* k;       // bf16 [n_seq][L][H][DK]
    const uint16_t* v;       // bf16 [n_seq][L][H][DV]
    const float* alpha;      // [n_seq][L][H]
    const float* beta;       // [n_seq][L][H]
    const float* s_init;     // [n_seq][H][DV][DK] float32, or null (zero state)
    float* s_out;            // [n_seq][H][DV][DK] float32 (the float32 form)
    uint16_t* planes;        // [max_requests][H][2][DV*DK] bf16 hi/lo in MFMA fragment order (the plane form)
    int32_t n_seq, H, L;
    int32_t slot[kMaxReqPerLaunch];  // plane form: request id of sequence i
};

// S0 as the step kernel's two bf16 planes: hi = rne(x), lo = rne(x - hi).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Returns hipErrorInvalidValue for unsupported (DK, DV).
hipError_t launch_prefill(int dk, int dv, bool planes, const PrefillParams& p, hipStream_t s);
hipError_t launch_fullstate_step(int dk, int dv, const FullStateParams& p, hipStream_t s);
hipError_t launch_replay_step(int dk, int dv, const ReplayParams& p, hipStream_t s);
hipError_t launch_init_s0(int dk, int dv, const float* S0, uint16_t* planes, int H, hipStream_t s);
// Which step bodies a launch needs: every request at its first step (no
// ancestral record to gather), none at its first step, or either (graph mode,
// where the step index is on the device, or requests at mixed depths).
constexpr int kStepFirst = 0, kStepHist = 1, kStepAny = 2;
// half_chunks: the general body takes kChunk / 2 beams per chunk (small
// launches; beams_per_block a multiple of kChunk / 2), else kChunk.
hipError_t launch_step(int dk, int dv, bool fused, int mode, bool half_chunks, const StepParams& p, hipStream_t s);
// Set the launch attributes the step kernel needs for this shape (once, before any launch).
hipError_t prepare_step(int dk, int dv, int T_max, int W);
// steps[req] = steps_value, epoch[req] = epoch_value (a request restarts).
hipError_t launch_set_counters(int32_t* dev_steps, int32_t* dev_epoch, int req, int steps_value, int epoch_value,
                               hipStream_t s);
bool step_supported(int dk, int dv);
size_t step_lds_bytes(int dk, int dv, int T_max, int W);

}  // namespace onela
