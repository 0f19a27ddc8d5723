// Measurement probes for bench.py (declared in onela_probes.h); not part of
// the decode path.
//
// copy:        plain 16-byte device copy, the practical HBM rate.
// mfma loop:   register-only 16x16x32 bf16 MFMAs, the practical matrix-core rate.
// planes:      S0 to the bf16 hi + lo planes in MFMA A-fragment order, the
//              form the step kernel holds its shared state in.
// projection:  P = S0 [k q] for every (request, head) pair with the step
//              kernel's tiling (wave w loads rows 16w..16w+15 of S0 from the
//              planes as A-fragments; k and q are staged through LDS 64 beams
//              at a time, the next chunk in flight during this chunk's MFMAs,
//              and read as B-fragments; two MFMAs per tile), reduced to
//              per-row sums over the beams so that nothing but the projection
//              is timed and the result can be checked (S0 times the sum of
//              the vectors, since the projection is linear).
#include <algorithm>

#include "../../include/onela_probes.h"
#include "onela_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// four 16-byte loads in flight per thread, then four stores (streaming hints)
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
    const size_t base = (size_t)blockIdx.x * 1024 + threadIdx.x;
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const size_t j = base + i * 256;
        if (j < n) v[i] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const size_t j = base + i * 256;
        if (j < n) __builtin_nontemporal_store(v[i], dst + j);
    }
}

__global__ __launch_bounds__(512) void mfma_loop_kernel(float* out, int iters) {
    // operands derived from the thread id, so the compiler cannot fold them
    const uint32_t t = threadIdx.x;
    u32x4 wa, wb;
    for (int e = 0; e < 4; ++e) {
        wa[e] = 0x3c003c00u ^ ((t * 2654435761u + e) & 0x007f007fu);
        wb[e] = 0x3c003c00u ^ ((t * 40503u + 7u * e) & 0x007f007fu);
    }
    const bf16x8 a = __builtin_bit_cast(bf16x8, wa), b = __builtin_bit_cast(bf16x8, wb);
    f32x4 acc[8];
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    out[(size_t)blockIdx.x * 512 + t] = s;
}

// fragment f = (w*4 + kk)*64 + lane of a pair's hi plane (then of its lo
// plane) holds S0[16w + lane%16][32kk + 8(lane/16) + 0..7], d_k = d_v = 128;
// hi = rne(S0), lo = rne(S0 - hi)
__global__ __launch_bounds__(256) void planes_kernel(const float* __restrict__ S0, uint16_t* __restrict__ planes,
                                                     int n_pairs) {
    constexpr int DK = 128, DV = 128, KS = DK / 32, NFRAG = DV * DK / 8;
    const int f = blockIdx.x * 256 + threadIdx.x;
    if (f >= n_pairs * NFRAG) return;
    const int pr = f / NFRAG, fi = f % NFRAG;
    const int lane = fi & 63, w = (fi >> 6) / KS, kk = (fi >> 6) % KS;
    const float* src = S0 + ((size_t)pr * DV + 16 * w + (lane & 15)) * DK + 32 * kk + 8 * (lane >> 4);
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    u32x4 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t h0 = onela::f32_to_bf16_rne(xv[2 * e]), h1 = onela::f32_to_bf16_rne(xv[2 * e + 1]);
        hi[e] = h0 | (h1 << 16);
        lo[e] = onela::f32_to_bf16_rne(xv[2 * e] - __uint_as_float(h0 << 16)) |
                (onela::f32_to_bf16_rne(xv[2 * e + 1] - __uint_as_float(h1 << 16)) << 16);
    }
    u32x4* out = reinterpret_cast<u32x4*>(planes + (size_t)pr * 2 * DV * DK);
    out[fi] = hi;
    out[NFRAG + fi] = lo;
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void projection_kernel(
    const uint16_t* __restrict__ planes, const uint16_t* __restrict__ k, const uint16_t* __restrict__ q, int H,
    int W, int resident, float* __restrict__ colsum) {
    constexpr int DK = 128, DV = 128, KS = DK / 32, CH = 64, XS = DK + 16, SEG = DK / 8;
    constexpr int PIECES = (2 * CH * SEG) / 512;     // 16-byte pieces of a chunk per thread
    __shared__ __align__(16) uint16_t xs[2][2 * CH * XS];   // two chunk buffers
    const int src = resident ? (int)(blockIdx.x % resident) : (int)blockIdx.x;   // pair whose operands are read
    const int ri = src / H, h = src % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, quad = lane >> 4;

    bf16x8 a_hi[KS], a_lo[KS];
    {
        const bf16x8* pl = reinterpret_cast<const bf16x8*>(planes + (size_t)src * 2 * DV * DK);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            a_hi[kk] = pl[(wave * KS + kk) * 64 + lane];
            a_lo[kk] = pl[DV * DK / 8 + (wave * KS + kk) * 64 + lane];
        }
    }

    const size_t in0 = (size_t)ri * W * H + h;     // input row of (beam 0, head h)
    // the next chunk's k and q rows are loaded while this chunk's MFMAs run
    u32x4 pre[PIECES];                               // (vector type: stays in registers)
    auto load_chunk = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < PIECES; ++it) {
            const int idx = tid + it * 512;
            const int row = idx / SEG, seg = idx % SEG;
            const bool is_k = row < CH;
            const size_t b = (size_t)c0 + (is_k ? row : row - CH);
            pre[it] = *reinterpret_cast<const u32x4*>((is_k ? k : q) + (in0 + b * H) * DK + seg * 8);
        }
    };
    auto stage_chunk = [&](uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < PIECES; ++it) {
            const int idx = tid + it * 512;
            *reinterpret_cast<u32x4*>(buf + (idx / SEG) * XS + (idx % SEG) * 8) = pre[it];
        }
    };
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
    load_chunk(0);
    stage_chunk(xs[0]);
    __syncthreads();
    for (int c0 = 0, cb = 0; c0 < W; c0 += CH, cb ^= 1) {
        // (unconditional, from a clamped chunk: a branch around the loads
        // would make the compiler wait for them right away)
        load_chunk(min(c0 + CH, W - CH));
        __builtin_amdgcn_sched_barrier(0);           // keep the loads ahead of the MFMAs
        const uint16_t* x = xs[cb];
#pragma unroll
        for (int g = 0; g < CH / 32; ++g) {
            f32x4 acc[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int col = (ct >= 2 ? CH : 0) + g * 32 + (ct & 1) * 16 + n16;
                    const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(x + col * XS + kk * 32 + quad * 8);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi[kk], bfr, acc[ct], 0, 0, 0);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo[kk], bfr, acc[ct], 0, 0, 0);
                }
            }
            tot += (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
        if (c0 + CH < W) stage_chunk(xs[cb ^ 1]);   // that buffer was last read before the previous barrier
        __syncthreads();
    }
    // accumulator register i of lane l holds row 4*(l/16) + i for the beams of column l%16:
    // sum over the 16 columns
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] += __shfl_xor(tot[i], m, 64);
    }
    if (n16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) colsum[(size_t)blockIdx.x * DV + 16 * wave + 4 * quad + i] = tot[i];
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" int32_t onela_probe_copy(const void* src, void* dst, size_t n16, void* hip_stream) {
    if (!src || !dst || !aligned16(src) || !aligned16(dst)) return -1;
    if (n16 == 0) return 0;
    const size_t blocks = (n16 + 1023) / 1024;
    if (blocks > 0x7fffffff) return -1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(hip_stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int32_t onela_probe_mfma(float* out, int32_t n_wg, int32_t iters, void* hip_stream) {
    if (!out || n_wg < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_wg), dim3(512), 0, static_cast<hipStream_t>(hip_stream), out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int32_t onela_probe_planes(const float* S0, uint16_t* planes, int32_t n_pairs, void* hip_stream) {
    if (!S0 || !planes || n_pairs < 1 || !aligned16(S0) || !aligned16(planes)) return -1;
    if ((int64_t)n_pairs * 2048 >= INT32_MAX) return -1;
    hipLaunchKernelGGL(planes_kernel, dim3(n_pairs * 8), dim3(256), 0, static_cast<hipStream_t>(hip_stream), S0,
                       planes, n_pairs);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int32_t onela_probe_projection(const uint16_t* planes, const uint16_t* k, const uint16_t* q,
                                          int32_t n_req, int32_t H, int32_t W, int32_t resident_pairs, float* colsum,
                                          void* hip_stream) {
    if (!planes || !k || !q || !colsum || n_req < 1 || H < 1 || W < 64 || W % 64 != 0) return -1;
    if (!aligned16(planes) || !aligned16(k) || !aligned16(q)) return -1;
    if ((int64_t)n_req * H >= INT32_MAX || resident_pairs < 0 || resident_pairs > n_req * H) return -1;
    hipLaunchKernelGGL(projection_kernel, dim3(n_req * H), dim3(512), 0, static_cast<hipStream_t>(hip_stream),
                       planes, k, q, H, W, resident_pairs, colsum);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
