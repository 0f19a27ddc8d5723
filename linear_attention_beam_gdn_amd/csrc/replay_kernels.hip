// gfx950 kernel of the replay comparator: the decode step as a replay-based
// serving path performs it.
//
// A replay-based path keeps a state checkpoint only at the prompt boundary
// and treats every beam as an independent request, replaying its own history
// to rebuild the state (OneLA review, evolve.pub, "Summary" and "Scope &
// Claims": the ReplaySSM baseline). Here each beam, at every step, starts
// from S0, applies its ancestral records oldest first,
//   S <- alpha_j S + delta_j k_j^T,
// and then takes the GDN step on its own full state, which is dropped
// afterwards: nothing is shared between beams (not even S0 k), no per-beam
// state persists. Row i of S only needs row i of S0 and the records, so the
// kernel streams rows as the full-state comparator does: d_k/8 threads per
// row, 8 floats each.
#include "onela_internal.h"

namespace onela {
namespace {

__device__ __forceinline__ float bf16v(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

template <int DK, int DV>
__host__ __device__ constexpr int rs_threads() { return (DK / 8) * DV < 256 ? (DK / 8) * DV : 256; }

template <int DK, int DV>
__global__ __launch_bounds__((rs_threads<DK, DV>())) void rs_step_kernel(const ReplayParams p) {
    constexpr int NT = rs_threads<DK, DV>();
    constexpr int TPR = DK / 8;              // threads per row (8 floats each)
    constexpr int RPI = NT / TPR;            // rows per pass of the workgroup
    constexpr int NPASS = DV / RPI;
    static_assert(DK % 8 == 0 && NT % TPR == 0 && DV % RPI == 0 && TPR <= 64, "row split");
    extern __shared__ int chain_s[];         // [T_max - 1]: ancestor beam at steps 1 .. t-1

    const int tid = threadIdx.x;
    const int seg = tid % TPR, rsub = tid / TPR;
    // one workgroup per (call-local request, head, beam)
    const int b = blockIdx.x % p.W;
    const int pair = blockIdx.x / p.W;
    const int ri = pair / p.H, h = pair % p.H;
    const int slot = p.slot[ri], t = p.t[ri];
    const int W = p.W;
    const size_t in_row = ((size_t)ri * W + b) * p.H + h;        // row of (beam, head) in the inputs
    const size_t SZ = (size_t)DV * DK;
    const size_t rec0 = ((size_t)slot * p.H + h) * (size_t)p.T_max * W;   // record 0 of this (request, head)
    int32_t* hist = p.par_hist + (size_t)slot * p.T_max * W;

    // the beam's ancestors, newest first: this step's parent, then the stored parents of older steps
    if (tid == 0 && t > 1) {
        int par = p.parent[(size_t)ri * W + b];
        if (par < 0 || par >= W) {
            p.err[slot] = p.epoch[ri];
            par = 0;
        }
        chain_s[t - 2] = par;
        for (int s = t - 2; s >= 1; --s) {
            int a = hist[(size_t)s * W + chain_s[s]];
            chain_s[s - 1] = (a < 0 || a >= W) ? 0 : a;      // (stored clamped by the step that wrote it)
        }
    }
    // one head stores this step's parents for the steps that follow
    if (h == 0 && tid == 0 && t > 1) {
        const int par = p.parent[(size_t)ri * W + b];
        hist[(size_t)(t - 1) * W + b] = (par < 0 || par >= W) ? 0 : par;
    }
    __syncthreads();

    // this thread's 8 columns of k and q
    const uint4 kb = *reinterpret_cast<const uint4*>(p.k + in_row * DK + seg * 8);
    const uint4 qb = *reinterpret_cast<const uint4*>(p.q + in_row * DK + seg * 8);
    float kc[8], qc[8];
    {
        const uint16_t* kh = reinterpret_cast<const uint16_t*>(&kb);
        const uint16_t* qh = reinterpret_cast<const uint16_t*>(&qb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kc[e] = bf16v(kh[e]);
            qc[e] = bf16v(qh[e]);
        }
    }
    const float a = p.alpha[in_row], bt = p.beta[in_row];
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) kq = fmaf(kc[e], qc[e], kq);
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) kq += __shfl_xor(kq, m, 64);

    // S0 rows of this thread
    float sv[NPASS][8];
    const float* s0 = p.s0 + ((size_t)slot * p.H + h) * SZ;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const float* r = s0 + (size_t)(ps * RPI + rsub) * DK + seg * 8;
        const float4 x0 = *reinterpret_cast<const float4*>(r);
        const float4 x1 = *reinterpret_cast<const float4*>(r + 4);
        sv[ps][0] = x0.x; sv[ps][1] = x0.y; sv[ps][2] = x0.z; sv[ps][3] = x0.w;
        sv[ps][4] = x1.x; sv[ps][5] = x1.y; sv[ps][6] = x1.z; sv[ps][7] = x1.w;
    }
    // replay the ancestral records, oldest first (record of step s: (s-1) W + ancestor)
    for (int s = 1; s < t; ++s) {
        const size_t rid = rec0 + (size_t)(s - 1) * W + chain_s[s - 1];
        const float aj = p.rec_alpha[rid];
        const uint4 kjb = *reinterpret_cast<const uint4*>(p.rec_k + rid * DK + seg * 8);
        const uint16_t* kjh = reinterpret_cast<const uint16_t*>(&kjb);
        float kj[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kj[e] = bf16v(kjh[e]);
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            const float dj = p.rec_delta[rid * DV + ps * RPI + rsub];
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[ps][e] = fmaf(aj, sv[ps][e], dj * kj[e]);
        }
    }
    // the step on the rebuilt state; the record is appended, the state dropped
    const size_t rnew = rec0 + (size_t)(t - 1) * W + b;
    if (tid == 0) p.rec_alpha[rnew] = a;
    if (rsub == 0) *reinterpret_cast<uint4*>(p.rec_k + rnew * DK + seg * 8) = kb;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ps * RPI + rsub;
        float u = 0.f, w = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            u = fmaf(sv[ps][e], kc[e], u);
            w = fmaf(sv[ps][e], qc[e], w);
        }
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1) {
            u += __shfl_xor(u, m, 64);
            w += __shfl_xor(w, m, 64);
        }
        const float d = bt * (bf16v(p.v[in_row * DV + row]) - a * u);
        if (seg == 0) {
            p.o[in_row * DV + row] = fmaf(a, w, kq * d);
            p.rec_delta[rnew * DV + row] = d;
            if (p.delta_out) p.delta_out[in_row * DV + row] = d;
        }
    }
}

template <int DK, int DV>
hipError_t launch_rs_t(const ReplayParams& p, hipStream_t s) {
    const size_t lds = sizeof(int) * (size_t)(p.T_max > 1 ? p.T_max - 1 : 1);
    hipLaunchKernelGGL((rs_step_kernel<DK, DV>), dim3(p.n_req * p.H * p.W), dim3(rs_threads<DK, DV>()), lds, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_replay_step(int dk, int dv, const ReplayParams& p, hipStream_t s) {
    if (dk == 32 && dv == 32) return launch_rs_t<32, 32>(p, s);
    if (dk == 64 && dv == 64) return launch_rs_t<64, 64>(p, s);
    if (dk == 128 && dv == 128) return launch_rs_t<128, 128>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace onela
