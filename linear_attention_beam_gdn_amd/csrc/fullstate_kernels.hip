// gfx950 kernel of the full-state comparator: the decode step OneLA replaces.
//
// Every beam keeps its own d_v x d_k float32 state (OneLA review, evolve.pub,
// "Summary" and "Scope & Claims": the FullState serving path materialises a
// full state per beam, Theta(W d_v d_k) memory and per-step traffic). A step
// reads the parent's state, applies the GDN update and writes the beam's new
// state. Row i of S only needs row i of the parent state:
//   u_i = S_i . k,  w_i = S_i . q,  delta_i = beta (v_i - alpha u_i),
//   S'_i = alpha S_i + delta_i k,  o_i = alpha w_i + (k . q) delta_i,
// so the kernel streams rows: d_k/8 threads per row, 8 floats each.
#include "onela_internal.h"

namespace onela {
namespace {

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

template <int DK, int DV>
__host__ __device__ constexpr int fs_threads() { return (DK / 8) * DV < 256 ? (DK / 8) * DV : 256; }

template <int DK, int DV>
__global__ __launch_bounds__((fs_threads<DK, DV>())) void fs_step_kernel(const FullStateParams p) {
    constexpr int NT = fs_threads<DK, DV>();
    constexpr int TPR = DK / 8;              // threads per row (8 floats each)
    constexpr int RPI = NT / TPR;            // rows per pass of the workgroup
    constexpr int NPASS = DV / RPI;
    static_assert(DK % 8 == 0 && NT % TPR == 0 && DV % RPI == 0 && TPR <= 64, "row split");

    const int tid = threadIdx.x;
    const int seg = tid % TPR, rsub = tid / TPR;
    // one workgroup per (call-local request, head, beam)
    const int b = blockIdx.x % p.W;
    const int pair = blockIdx.x / p.W;
    const int ri = pair / p.H, h = pair % p.H;
    const int slot = p.slot[ri], t = p.t[ri];
    const size_t in_row = ((size_t)ri * p.W + b) * p.H + h;       // row of (beam, head) in the inputs
    const size_t SZ = (size_t)DV * DK;

    const float* src;
    if (t == 1) {
        src = p.s0 + ((size_t)slot * p.H + h) * SZ;
    } else {
        int par = p.parent[(size_t)ri * p.W + b];
        if (par < 0 || par >= p.W) {
            p.err[slot] = p.epoch[ri];
            par = 0;
        }
        src = p.state + ((((size_t)((t - 1) & 1) * p.max_requests + slot) * p.H + h) * p.W + par) * SZ;
    }
    float* dst = p.state + ((((size_t)(t & 1) * p.max_requests + slot) * p.H + h) * p.W + b) * SZ;

    // this thread's 8 columns of k and q
    const uint4 kb = *reinterpret_cast<const uint4*>(p.k + in_row * DK + seg * 8);
    const uint4 qb = *reinterpret_cast<const uint4*>(p.q + in_row * DK + seg * 8);
    float kc[8], qc[8];
    {
        const uint16_t* kh = reinterpret_cast<const uint16_t*>(&kb);
        const uint16_t* qh = reinterpret_cast<const uint16_t*>(&qb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kc[e] = bf16f(kh[e]);
            qc[e] = bf16f(qh[e]);
        }
    }
    const float a = p.alpha[in_row], bt = p.beta[in_row];
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) kq = fmaf(kc[e], qc[e], kq);
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) kq += __shfl_xor(kq, m, 64);

    // all rows of this thread in flight at once
    float4 s[NPASS][2];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const float* r = src + (size_t)(ps * RPI + rsub) * DK + seg * 8;
        s[ps][0] = *reinterpret_cast<const float4*>(r);
        s[ps][1] = *reinterpret_cast<const float4*>(r + 4);
    }
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ps * RPI + rsub;
        const float sv[8] = {s[ps][0].x, s[ps][0].y, s[ps][0].z, s[ps][0].w,
                             s[ps][1].x, s[ps][1].y, s[ps][1].z, s[ps][1].w};
        float u = 0.f, w = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            u = fmaf(sv[e], kc[e], u);
            w = fmaf(sv[e], qc[e], w);
        }
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1) {
            u += __shfl_xor(u, m, 64);
            w += __shfl_xor(w, m, 64);
        }
        const float d = bt * (bf16f(p.v[in_row * DV + row]) - a * u);
        float nv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) nv[e] = fmaf(a, sv[e], d * kc[e]);
        float* wr = dst + (size_t)row * DK + seg * 8;
        *reinterpret_cast<float4*>(wr) = make_float4(nv[0], nv[1], nv[2], nv[3]);
        *reinterpret_cast<float4*>(wr + 4) = make_float4(nv[4], nv[5], nv[6], nv[7]);
        if (seg == 0) {
            p.o[in_row * DV + row] = fmaf(a, w, kq * d);
            if (p.delta_out) p.delta_out[in_row * DV + row] = d;
        }
    }
}

template <int DK, int DV>
hipError_t launch_fs_t(const FullStateParams& p, hipStream_t s) {
    hipLaunchKernelGGL((fs_step_kernel<DK, DV>), dim3(p.n_req * p.H * p.W), dim3(fs_threads<DK, DV>()), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fullstate_step(int dk, int dv, const FullStateParams& p, hipStream_t s) {
    if (dk == 32 && dv == 32) return launch_fs_t<32, 32>(p, s);
    if (dk == 64 && dv == 64) return launch_fs_t<64, 64>(p, s);
    if (dk == 128 && dv == 128) return launch_fs_t<128, 128>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace onela
