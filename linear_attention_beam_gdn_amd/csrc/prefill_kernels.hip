// gfx950 kernel of the prefill: the prompt-derived state decoding starts from.
//
// Every request's beams share one state obtained by running the GDN
// recurrence over the prompt (OneLA abstract: a single shared prompt-derived
// state; OneLA review, evolve.pub, paper Eq. 2: the GDN recurrence). For
// prompt tokens s = 1..L of one (sequence, head):
//   u = S k_s,  delta = beta_s (v_s - alpha_s u),  S <- alpha_s S + delta k_s^T.
// One workgroup per (sequence, head) keeps S in registers for the whole
// prompt: each lane holds a quarter of the columns of two rows. Tokens are staged in
// LDS (as float32) kTokBlock at a time; the next block's loads are in flight
// while the current block is folded. Within a block S is held as S / c with
// c the block's running decay, so a token costs two multiply-adds per state
// element. The result is written either as float32 [H][d_v][d_k] or directly
// as the step kernel's two bf16 planes.
#include "onela_internal.h"

namespace onela {
namespace {

constexpr int kTokBlock = 16;   // prompt tokens staged per block

template <int DV>
__host__ __device__ constexpr int prefill_threads() { return 2 * DV; }

template <int DK, int DV, bool PLANES>
__global__ __launch_bounds__(prefill_threads<DV>()) void prefill_kernel(const PrefillParams p) {
    constexpr int NT = prefill_threads<DV>();
    constexpr int C = DK / 4;            // state columns per thread (a quarter of each of its two rows)
    constexpr int TB = kTokBlock;
    constexpr int KP = DK / 8, VP = DV / 8;   // 16-byte pieces per token row
    // one k piece and one v piece of a block per thread; four lanes per row pair
    static_assert(TB * KP == NT && TB * VP == NT && C % 8 == 0 && NT == 2 * DV, "prefill block shape");

    __shared__ __align__(16) float ks[2][TB][DK];
    __shared__ __align__(16) float vsh[2][TB][DV];
    __shared__ float as[2][TB], bs[2][TB];

    const int tid = threadIdx.x;
    // rows r, r + DV/2 (r = tid / 4), columns [cq*C, cq*C + C) with cq = tid % 4
    const int cq = tid & 3;
    const int rows[2] = {tid >> 2, (tid >> 2) + DV / 2};
    const int seq = blockIdx.x / p.H, h = blockIdx.x % p.H;
    const int H = p.H, L = p.L;
    const size_t tok0 = (size_t)seq * L;                 // token 0 of this sequence
    const size_t state0 = ((size_t)seq * H + h) * DV * DK;

    float S[2][C];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (p.s_init) {
            const float4* src = reinterpret_cast<const float4*>(p.s_init + state0 + (size_t)rows[q] * DK + cq * C);
#pragma unroll
            for (int j = 0; j < C / 4; ++j) {
                const float4 x = src[j];
                S[q][4 * j] = x.x; S[q][4 * j + 1] = x.y; S[q][4 * j + 2] = x.z; S[q][4 * j + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < C; ++j) S[q][j] = 0.f;
        }
    }

    // this thread's pieces of a block: token tid / KP, 8 bf16 values at (tid % KP) * 8
    const int lt = tid / KP, kpc = (tid % KP) * 8;
    const int vt = tid / VP, vpc = (tid % VP) * 8;
    uint4 kreg = make_uint4(0, 0, 0, 0), vreg = make_uint4(0, 0, 0, 0);
    float abreg = 0.f;
    auto load_block = [&](int s0) __attribute__((always_inline)) {
        const size_t sk = tok0 + min(s0 + lt, L - 1);    // clamped: tail tokens are never folded
        const size_t sv = tok0 + min(s0 + vt, L - 1);
        kreg = *reinterpret_cast<const uint4*>(p.k + (sk * H + h) * DK + kpc);
        vreg = *reinterpret_cast<const uint4*>(p.v + (sv * H + h) * DV + vpc);
        const size_t sa = tok0 + min(s0 + (tid % TB), L - 1);
        abreg = (tid < TB ? p.alpha : p.beta)[sa * H + h];   // threads 0..TB-1 alpha, TB..2TB-1 beta
    };
    auto stage_block = [&](int buf) __attribute__((always_inline)) {
        const uint32_t kw[4] = {kreg.x, kreg.y, kreg.z, kreg.w};
        const uint32_t vw[4] = {vreg.x, vreg.y, vreg.z, vreg.w};
        float kf[8], vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kf[2 * e] = __uint_as_float(kw[e] << 16);
            kf[2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
            vf[2 * e] = __uint_as_float(vw[e] << 16);
            vf[2 * e + 1] = __uint_as_float(vw[e] & 0xffff0000u);
        }
        float4* kd = reinterpret_cast<float4*>(&ks[buf][lt][kpc]);
        kd[0] = make_float4(kf[0], kf[1], kf[2], kf[3]);
        kd[1] = make_float4(kf[4], kf[5], kf[6], kf[7]);
        float4* vd = reinterpret_cast<float4*>(&vsh[buf][vt][vpc]);
        vd[0] = make_float4(vf[0], vf[1], vf[2], vf[3]);
        vd[1] = make_float4(vf[4], vf[5], vf[6], vf[7]);
        if (tid < TB) as[buf][tid] = abreg;
        else if (tid < 2 * TB) bs[buf][tid - TB] = abreg;
    };

    const int nblk = (L + TB - 1) / TB;
    if (nblk > 0) {
        load_block(0);
        stage_block(0);
    }
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
        const int buf = blk & 1;
        if (blk + 1 < nblk) load_block((blk + 1) * TB);   // in flight while this block is folded
        const int ntok = min(TB, L - blk * TB);
        // Within a block the registers hold S / c, with c the product of the
        // block's decays so far: the decay then costs one multiply per token
        // instead of one per state element, and the update is a single
        // multiply-add per element. c is folded back in at the end of every
        // block (and early, should it leave [2^-60, 2^60]).
        float c = 1.f;
        for (int tk = 0; tk < ntok; ++tk) {
            float kr[C];
            const float4* kt = reinterpret_cast<const float4*>(&ks[buf][tk][cq * C]);
#pragma unroll
            for (int j = 0; j < C / 4; ++j) {
                const float4 x = kt[j];
                kr[4 * j] = x.x; kr[4 * j + 1] = x.y; kr[4 * j + 2] = x.z; kr[4 * j + 3] = x.w;
            }
            float u[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float acc[2] = {0.f, 0.f};
#pragma unroll
                for (int j = 0; j < C; ++j) acc[j & 1] = fmaf(S[q][j], kr[j], acc[j & 1]);
                u[q] = acc[0] + acc[1];
                // the row's other quarters sit in the lanes of the same quad
                u[q] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(u[q]), 0xB1, 0xF, 0xF, true));  // lane ^ 1
                u[q] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(u[q]), 0x4E, 0xF, 0xF, true));  // lane ^ 2
            }
            const float a = as[buf][tk], bt = bs[buf][tk];
            const float d0 = bt * (vsh[buf][tk][rows[0]] - a * (u[0] * c));   // u * c = S k
            const float d1 = bt * (vsh[buf][tk][rows[1]] - a * (u[1] * c));
            c *= a;                                              // S' = c (S/c_prev + (d / c) k^T)
            if (!(c >= 0x1p-60f && c <= 0x1p60f)) {              // (uniform) fold the scale in early
#pragma unroll
                for (int j = 0; j < C; ++j) {
                    S[0][j] *= c;
                    S[1][j] *= c;
                }
                c = 1.f;
            }
            const float rc = 1.f / c;
            const float dc0 = d0 * rc, dc1 = d1 * rc;
#pragma unroll
            for (int j = 0; j < C; ++j) {
                S[0][j] = fmaf(dc0, kr[j], S[0][j]);
                S[1][j] = fmaf(dc1, kr[j], S[1][j]);
            }
        }
#pragma unroll
        for (int j = 0; j < C; ++j) {
            S[0][j] *= c;
            S[1][j] *= c;
        }
        if (blk + 1 < nblk) stage_block(buf ^ 1);   // the other buffer was last read before the previous barrier
        __syncthreads();
    }

#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = rows[q];
        if (!PLANES) {
            float4* dst = reinterpret_cast<float4*>(p.s_out + state0 + (size_t)row * DK + cq * C);
#pragma unroll
            for (int j = 0; j < C / 4; ++j)
                dst[j] = make_float4(S[q][4 * j], S[q][4 * j + 1], S[q][4 * j + 2], S[q][4 * j + 3]);
        } else {
            // fragment f = (w*KS + kk)*64 + lane holds S[16w + lane%16][32kk + 8(lane/16) + 0..7]
            constexpr int KS = DK / 32;
            uint16_t* pl = p.planes + ((size_t)p.slot[seq] * H + h) * 2 * DV * DK;
            const int w = row / 16;
#pragma unroll
            for (int g8 = 0; g8 < C / 8; ++g8) {
                const int col = cq * C + g8 * 8;
                const int kk = col / 32, lane = (row % 16) + 16 * ((col % 32) / 8);
                const size_t f = ((size_t)w * KS + kk) * 64 + lane;
                uint32_t hi[8], lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    hi[e] = f32_to_bf16_rne(S[q][g8 * 8 + e]);
                    lo[e] = f32_to_bf16_rne(S[q][g8 * 8 + e] - __uint_as_float(hi[e] << 16));
                }
                *reinterpret_cast<uint4*>(pl + f * 8) = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                                                                   hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
                *reinterpret_cast<uint4*>(pl + DV * DK + f * 8) = make_uint4(
                    lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
            }
        }
    }
}

template <int DK, int DV>
hipError_t launch_prefill_t(bool planes, const PrefillParams& p, hipStream_t s) {
    const dim3 grid(p.n_seq * p.H), block(prefill_threads<DV>());
    if (planes)
        hipLaunchKernelGGL((prefill_kernel<DK, DV, true>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((prefill_kernel<DK, DV, false>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(int dk, int dv, bool planes, const PrefillParams& p, hipStream_t s) {
    if (dk == 32 && dv == 32) return launch_prefill_t<32, 32>(planes, p, s);
    if (dk == 64 && dv == 64) return launch_prefill_t<64, 64>(planes, p, s);
    if (dk == 128 && dv == 128) return launch_prefill_t<128, 128>(planes, p, s);
    return hipErrorInvalidValue;
}

}  // namespace onela
