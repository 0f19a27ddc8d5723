// gfx950 kernels of the OneLA large-beam GDN decode step.
//
// One launch per decode step of one GDN layer (OneLA abstract: a fused GPU
// kernel reuses the shared state across beams). A workgroup owns one
// (request, head) pair and a range of beams, which it walks in chunks of
// kChunk beams. For each chunk it
//   A. stages k_t and q_t of the chunk's beams in LDS, appends k_t and
//      alpha_t to the record store, and builds each beam's ancestry row from
//      its parent's row (ids only; OneLA abstract: records are never moved);
//   B. computes, per beam and ancestral record j, the dot products k_j . k_t
//      and k_j . q_t (the only way the replay touches x; OneLA review,
//      "Scope & Claims", paper Eq. 3), plus k_t . q_t;
//   C. projects the shared state once for all 2*kChunk vectors,
//      P = S0 [k_t q_t], on the matrix cores (split-bf16: S0 = hi + lo);
//   D. replays the ancestry in the MFMA accumulator registers,
//      y <- alpha_j y + (k_j . x) delta_j, which leaves y = S_{t-1} x, then
//      forms delta_t = beta (v - alpha y_k), o_t = alpha y_q + (k_t . q_t) delta_t
//      (= S_t q_t) and appends delta_t.
//
// Wave w of the workgroup owns rows [32w, 32w+32) of d_v: its slice of S0
// stays in registers as MFMA A-fragments for the whole beam loop, and every
// step after the projection is row-separable, so no wave ever needs another
// wave's rows.
#include "onela_internal.h"

namespace onela {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float dot8(uint4 a, uint4 b, float acc) {
    acc = fmaf(bf_lo(a.x), bf_lo(b.x), acc);
    acc = fmaf(bf_hi(a.x), bf_hi(b.x), acc);
    acc = fmaf(bf_lo(a.y), bf_lo(b.y), acc);
    acc = fmaf(bf_hi(a.y), bf_hi(b.y), acc);
    acc = fmaf(bf_lo(a.z), bf_lo(b.z), acc);
    acc = fmaf(bf_hi(a.z), bf_hi(b.z), acc);
    acc = fmaf(bf_lo(a.w), bf_lo(b.w), acc);
    acc = fmaf(bf_hi(a.w), bf_hi(b.w), acc);
    return acc;
}

// ---------------------------------------------------------------------------
// S0 (float32, row-major [H][DV][DK]) -> two bf16 planes hi, lo with
// hi = rne(S0), lo = rne(S0 - hi), stored in the order the step kernel loads
// its MFMA A-fragments: fragment f = (w*KS + kk)*64 + lane holds the 8 values
// S0[32w + lane%32][16kk + 8*(lane/32) + 0..7].
template <int DK, int DV>
__global__ __launch_bounds__(256) void init_s0_kernel(const float* __restrict__ S0,
                                                      uint16_t* __restrict__ planes, int H) {
    constexpr int KS = DK / 16;
    constexpr int NFRAG = DV * DK / 8;
    const int f = blockIdx.x * 256 + threadIdx.x;
    if (f >= H * NFRAG) return;
    const int h = f / NFRAG, fi = f % NFRAG;
    const int lane = fi & 63, wk = fi >> 6;
    const int w = wk / KS, kk = wk % KS;
    const int m = 32 * w + (lane & 31);
    const int kb = 16 * kk + 8 * (lane >> 5);
    const float* src = S0 + ((size_t)h * DV + m) * DK + kb;
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi[e] = f32_to_bf16_rne(xv[e]);
        lo[e] = f32_to_bf16_rne(xv[e] - __uint_as_float(hi[e] << 16));
    }
    uint16_t* ph = planes + (size_t)h * 2 * DV * DK + (size_t)fi * 8;
    *reinterpret_cast<uint4*>(ph) =
        make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
    *reinterpret_cast<uint4*>(ph + DV * DK) =
        make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
}

// ---------------------------------------------------------------------------
template <int DK>
__host__ __device__ constexpr int xs_row() { return DK + 8; }  // padded LDS row (bf16), breaks bank aliasing

template <int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 32)) void step_kernel(const StepParams p) {
    constexpr int CH = kChunk;
    constexpr int NW = DV / 32;        // waves; wave w owns d_v rows [32w, 32w+32)
    constexpr int NT = 64 * NW;
    constexpr int KS = DK / 16;        // MFMA k-steps
    constexpr int NB = CH / 32;        // 32-beam column groups per chunk
    constexpr int XS = xs_row<DK>();
    constexpr int TPB = NT / CH;       // threads per beam in the dot-product phase
    constexpr int EPT = DK / TPB;      // key elements per thread there
    static_assert(DV % 32 == 0 && DK % 16 == 0, "tile shape");
    static_assert(TPB >= 1 && EPT % 8 == 0, "dot-product split");

    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int MS = p.T_max > 1 ? p.T_max - 1 : 1;                  // ancestry depth capacity
    float4* coef_s = reinterpret_cast<float4*>(lds_raw);            // [CH][MS] {k_j.k_t, k_j.q_t, alpha_j, rid}
    uint16_t* xs = reinterpret_cast<uint16_t*>(coef_s + CH * MS);   // [2*CH][XS]: k rows then q rows
    int* anc_s = reinterpret_cast<int*>(xs + 2 * CH * XS);          // [CH][MS]
    float* kq_s = reinterpret_cast<float*>(anc_s + CH * MS);        // [CH]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Workgroups are dealt to the 8 XCDs round-robin; renumber them so that
    // the beam splits of one (request, head) land on one XCD and share its L2.
    int L = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) L = (L & 7) * (nblk >> 3) + (L >> 3);
    const int split = L % p.n_splits;
    const int pair = L / p.n_splits;
    const int ri = pair / p.H;
    const int h = pair % p.H;
    const int slot = p.slot[ri];
    const int t = p.t[ri];
    const int H = p.H, W = p.W;
    const int depth = t - 1;                      // ancestral records per beam
    const int b_begin = split * p.beams_per_block;
    const int b_end = min(W, b_begin + p.beams_per_block);
    if (b_begin >= b_end) return;

    const size_t pair_id = (size_t)slot * H + h;
    const size_t rec0 = pair_id * (size_t)p.T_max * W;            // record 0 of this (request, head)
    const size_t row0 = (size_t)ri * W;                            // first input row of this request
    const int* anc_prev = p.anc + ((size_t)((t - 1) & 1) * p.max_requests + slot) * (size_t)W * p.T_max;
    int* anc_next = p.anc + ((size_t)(t & 1) * p.max_requests + slot) * (size_t)W * p.T_max;

    // This wave's rows of S0 as A-fragments, resident for the whole beam loop.
    bf16x8 a_hi[KS], a_lo[KS];
    {
        const bf16x8* pl = reinterpret_cast<const bf16x8*>(p.s0_planes + pair_id * 2 * DV * DK);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            a_hi[kk] = pl[(wave * KS + kk) * 64 + lane];
            a_lo[kk] = pl[DV * DK / 8 + (wave * KS + kk) * 64 + lane];
        }
    }

    for (int c0 = b_begin; c0 < b_end; c0 += CH) {
        const int nb = min(CH, b_end - c0);

        // ---- A. stage k_t, q_t; append k_t, alpha_t; ancestry rows --------
        constexpr int SEG = DK / 8;                      // 16-byte pieces per row
        for (int idx = tid; idx < 2 * CH * SEG; idx += NT) {
            const int row = idx / SEG, seg = idx % SEG;
            const bool is_k = row < CH;
            const int bl = is_k ? row : row - CH;
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (bl < nb) {
                const size_t in = ((row0 + c0 + bl) * H + h) * DK + seg * 8;
                val = *reinterpret_cast<const uint4*>((is_k ? p.k : p.q) + in);
                if (is_k)
                    *reinterpret_cast<uint4*>(p.rec_k + (rec0 + (size_t)depth * W + c0 + bl) * DK + seg * 8) = val;
            }
            *reinterpret_cast<uint4*>(xs + row * XS + seg * 8) = val;
        }
        for (int bl = tid; bl < nb; bl += NT) {
            const int b = c0 + bl;
            p.rec_alpha[rec0 + (size_t)depth * W + b] = p.alpha[(row0 + b) * H + h];
            if (depth > 0) {
                int par = p.parent[row0 + b];
                if (par < 0 || par >= W) {        // reported through the error word
                    p.err[slot] = p.epoch[ri];
                    par = 0;
                }
                const int* src = anc_prev + (size_t)par * p.T_max;
                for (int j = 0; j + 1 < depth; ++j) anc_s[bl * MS + j] = src[j];
                anc_s[bl * MS + depth - 1] = (depth - 1) * W + par;   // parent's own record of step t-1
                if (h == 0)   // one head writes the request's new index rows
                    for (int j = 0; j < depth; ++j) anc_next[(size_t)b * p.T_max + j] = anc_s[bl * MS + j];
            }
        }
        __syncthreads();

        // ---- B. dot products of the ancestral keys with k_t and q_t -------
        {
            const int bl = tid / TPB, part = tid % TPB;
            if (bl < nb) {
                uint4 kt[EPT / 8], qt[EPT / 8];
#pragma unroll
                for (int s = 0; s < EPT / 8; ++s) {
                    kt[s] = *reinterpret_cast<const uint4*>(xs + bl * XS + part * EPT + s * 8);
                    qt[s] = *reinterpret_cast<const uint4*>(xs + (CH + bl) * XS + part * EPT + s * 8);
                }
                float kq = 0.f;
#pragma unroll
                for (int s = 0; s < EPT / 8; ++s) kq = dot8(kt[s], qt[s], kq);
#pragma unroll
                for (int m = 1; m < TPB; m <<= 1) kq += __shfl_xor(kq, m, 64);
                if (part == 0) kq_s[bl] = kq;
                for (int j = 0; j < depth; ++j) {
                    const int r = anc_s[bl * MS + j];
                    const uint4* kj = reinterpret_cast<const uint4*>(p.rec_k + (rec0 + r) * DK + part * EPT);
                    float dk = 0.f, dq = 0.f;
#pragma unroll
                    for (int s = 0; s < EPT / 8; ++s) {
                        const uint4 kv = kj[s];
                        dk = dot8(kv, kt[s], dk);
                        dq = dot8(kv, qt[s], dq);
                    }
#pragma unroll
                    for (int m = 1; m < TPB; m <<= 1) {
                        dk += __shfl_xor(dk, m, 64);
                        dq += __shfl_xor(dq, m, 64);
                    }
                    if (part == 0) coef_s[bl * MS + j] = make_float4(dk, dq, p.rec_alpha[rec0 + r], __int_as_float(r));
                }
            }
        }

        __syncthreads();   // coef_s / kq_s complete

        // ---- C + D, one 32-beam group at a time ------------------------------
        // C: y_k = S0 k_t, y_q = S0 q_t for the group's 32 beams on the matrix
        //    cores (S0 = hi + lo, both bf16, fp32 accumulation).
        // D: replay, epilogue and append. Accumulator register 4*rr + e of
        //    lane l holds row 8*rr + 4*(l/32) + e (of this wave's 32) for
        //    column (beam) l%32.
        const int rbase = wave * 32 + (lane >> 5) * 4;
#pragma unroll
        for (int g = 0; g < NB; ++g) {
            const int bl = g * 32 + (lane & 31);
            f32x16 yk = f32x16{}, yq = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const int koff = kk * 16 + (lane >> 5) * 8;
                const bf16x8 bk = *reinterpret_cast<const bf16x8*>(xs + bl * XS + koff);
                const bf16x8 bq = *reinterpret_cast<const bf16x8*>(xs + (CH + bl) * XS + koff);
                yk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[kk], bk, yk, 0, 0, 0);
                yq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[kk], bq, yq, 0, 0, 0);
                yk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo[kk], bk, yk, 0, 0, 0);
                yq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo[kk], bq, yq, 0, 0, 0);
            }
            if (bl < nb) {
                for (int j = 0; j < depth; ++j) {
                    const float4 c = coef_s[bl * MS + j];
                    const float* dj = p.rec_delta + (rec0 + __float_as_int(c.w)) * DV + rbase;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const float4 d = *reinterpret_cast<const float4*>(dj + 8 * rr);
                        yk[4 * rr + 0] = fmaf(c.z, yk[4 * rr + 0], c.x * d.x);
                        yk[4 * rr + 1] = fmaf(c.z, yk[4 * rr + 1], c.x * d.y);
                        yk[4 * rr + 2] = fmaf(c.z, yk[4 * rr + 2], c.x * d.z);
                        yk[4 * rr + 3] = fmaf(c.z, yk[4 * rr + 3], c.x * d.w);
                        yq[4 * rr + 0] = fmaf(c.z, yq[4 * rr + 0], c.y * d.x);
                        yq[4 * rr + 1] = fmaf(c.z, yq[4 * rr + 1], c.y * d.y);
                        yq[4 * rr + 2] = fmaf(c.z, yq[4 * rr + 2], c.y * d.z);
                        yq[4 * rr + 3] = fmaf(c.z, yq[4 * rr + 3], c.y * d.w);
                    }
                }
                const int b = c0 + bl;
                const size_t row = (row0 + b) * H + h;
                const float at = p.alpha[row], bt = p.beta[row], kq = kq_s[bl];
                const uint16_t* vp = p.v + row * DV + rbase;
                float* op = p.o + row * DV + rbase;
                float* rp = p.rec_delta + (rec0 + (size_t)depth * W + b) * DV + rbase;
                float* dp = p.delta_out ? p.delta_out + row * DV + rbase : nullptr;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const uint2 vb = *reinterpret_cast<const uint2*>(vp + 8 * rr);
                    float4 d, o;
                    d.x = bt * (bf_lo(vb.x) - at * yk[4 * rr + 0]);
                    d.y = bt * (bf_hi(vb.x) - at * yk[4 * rr + 1]);
                    d.z = bt * (bf_lo(vb.y) - at * yk[4 * rr + 2]);
                    d.w = bt * (bf_hi(vb.y) - at * yk[4 * rr + 3]);
                    o.x = fmaf(at, yq[4 * rr + 0], kq * d.x);
                    o.y = fmaf(at, yq[4 * rr + 1], kq * d.y);
                    o.z = fmaf(at, yq[4 * rr + 2], kq * d.z);
                    o.w = fmaf(at, yq[4 * rr + 3], kq * d.w);
                    *reinterpret_cast<float4*>(op + 8 * rr) = o;
                    *reinterpret_cast<float4*>(rp + 8 * rr) = d;
                    if (dp) *reinterpret_cast<float4*>(dp + 8 * rr) = d;
                }
            }
        }
        __syncthreads();   // LDS is reused by the next chunk
    }
}

template <int DK, int DV>
hipError_t launch_init_t(const float* S0, uint16_t* planes, int H, hipStream_t s) {
    const int n = H * DV * DK / 8;
    hipLaunchKernelGGL((init_s0_kernel<DK, DV>), dim3((n + 255) / 256), dim3(256), 0, s, S0, planes, H);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_step_t(const StepParams& p, hipStream_t s) {
    const size_t lds = step_lds_bytes(DK, p.T_max);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&step_kernel<DK, DV>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int nblk = p.n_req * p.H * p.n_splits;
    hipLaunchKernelGGL((step_kernel<DK, DV>), dim3(nblk), dim3(64 * (DV / 32)), lds, s, p);
    return hipGetLastError();
}

}  // namespace

size_t step_lds_bytes(int dk, int T_max) {
    const size_t ms = T_max > 1 ? (size_t)T_max - 1 : 1;
    return kChunk * ms * 16 + 2 * kChunk * (size_t)(dk + 8) * 2 + kChunk * ms * 4 + kChunk * 4;
}

bool step_supported(int dk, int dv) {
    return dk == dv && (dk == 32 || dk == 64 || dk == 128);
}

hipError_t launch_init_s0(int dk, int dv, const float* S0, uint16_t* planes, int H, hipStream_t s) {
    if (dk == 32 && dv == 32) return launch_init_t<32, 32>(S0, planes, H, s);
    if (dk == 64 && dv == 64) return launch_init_t<64, 64>(S0, planes, H, s);
    if (dk == 128 && dv == 128) return launch_init_t<128, 128>(S0, planes, H, s);
    return hipErrorInvalidValue;
}

hipError_t launch_step(int dk, int dv, const StepParams& p, hipStream_t s) {
    if (dk == 32 && dv == 32) return launch_step_t<32, 32>(p, s);
    if (dk == 64 && dv == 64) return launch_step_t<64, 64>(p, s);
    if (dk == 128 && dv == 128) return launch_step_t<128, 128>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace onela
