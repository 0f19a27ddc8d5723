// gfx950 kernel of the prefill: the prompt-derived state decoding starts from.
//
// Every request's beams share one state obtained by running the GDN
// recurrence over the prompt (OneLA abstract: a single shared prompt-derived
// state; OneLA review, evolve.pub, paper Eq. 2: the GDN recurrence). For
// prompt tokens i of one (sequence, head):
//   delta_i = beta_i (v_i - alpha_i S_{i-1} k_i),  S_i = alpha_i S_{i-1} + delta_i k_i^T.
//
// Chunked form, 16 tokens at a time (one MFMA tile). With S the state before
// the chunk, g_i = alpha_1 ... alpha_i and r_ij = alpha_{j+1} ... alpha_i,
// unrolling the recurrence inside the chunk gives
//   delta_i = beta_i v_i - beta_i g_i S k_i - beta_i sum_{j<i} r_ij (k_i . k_j) delta_j,
// i.e. (I + L) Delta = RHS with L_ij = beta_i r_ij (k_i . k_j) (j < i) and
// RHS_i = beta_i (v_i - g_i S k_i), and the state after the chunk is
//   S' = g_16 S + sum_j r_16j delta_j k_j^T.
// T = (I + L)^-1 depends only on the chunk's keys and gates, so it is formed
// for several chunks at once before the state-dependent part runs. Per chunk
// the state-dependent part is three small products on the matrix cores:
//   P = K S^T (16 x d_v), Delta = T RHS, S'^T = g_16 S^T + K^T diag(r_16.) Delta,
// with the state held as float32 accumulators of S^T (wave w owns columns
// [16w, 16w+16) of S^T, i.e. rows of S) and every float32 operand split into
// bf16 hi + lo (keys are exact in bf16), the hi and lo halves folded into the
// 32-wide contraction of one 16x16x32 product. The accumulator layout of one
// product is the operand layout of the next, so nothing is reshuffled between
// them. A prompt folded in two calls is bit-identical to one call when the first
// part is a whole number of 16-token chunks.
#include "onela_internal.h"

namespace onela {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 16;        // tokens per chunk (one 16x16x16 MFMA tile)
constexpr int kTokBlock = 64;   // tokens staged in LDS at a time
constexpr int kSubPerBlock = kTokBlock / kSub;

template <int DV>
__host__ __device__ constexpr int prefill_threads() { return 64 * (DV / 16); }

// float32 -> bf16 hi + lo (round to nearest even), four at a time, two per conversion
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split4(f32x4 x, s16x4& hi, s16x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
        const f32x2 v = f32x2{x[e], x[e + 1]};
        const bf16x2v h = __builtin_convertvector(v, bf16x2v);
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const f32x2 hf = f32x2{__uint_as_float(hb << 16), __uint_as_float(hb & 0xffff0000u)};
        const bf16x2v l = __builtin_convertvector(v - hf, bf16x2v);
        const s16x2 hs = __builtin_bit_cast(s16x2, h), ls = __builtin_bit_cast(s16x2, l);
        hi[e] = hs[0]; hi[e + 1] = hs[1];
        lo[e] = ls[0]; lo[e + 1] = ls[1];
    }
}

// 16x16x32 product: lane l gives A[l%16][8(l/16) + e] and B[8(l/16) + e][l%16]
// (e = 0..7) and holds D[4(l/16) + r][l%16]. The contraction order is free, so
// a lane's eight k-slots carry either eight consecutive k or, to fold a bf16
// hi + lo pair into one product, the same four k twice: A's four values
// repeated against B's hi four then lo four.
__device__ __forceinline__ f32x4 mfma32(s16x8 a, s16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ s16x8 twice(s16x4 x) { return s16x8{x[0], x[1], x[2], x[3], x[0], x[1], x[2], x[3]}; }

__device__ __forceinline__ s16x8 cat(s16x4 x, s16x4 y) { return s16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]}; }

template <int DK, int DV, bool PLANES>
__global__ __launch_bounds__(prefill_threads<DV>(), DV >= 128 ? 4 : 1) void prefill_kernel(const PrefillParams p) {
    constexpr int NW = DV / 16;              // waves; wave w owns state rows [16w, 16w+16)
    constexpr int NT = 64 * NW;
    constexpr int KC = DK / 16;              // 16-wide column tiles of the state
    constexpr int TB = kTokBlock, NSC = kSubPerBlock;
    constexpr int KR = DK + 8;               // LDS row of a token's key (bf16)
    constexpr int TR = TB + 8;               // LDS row of a key / value column over the block's tokens (bf16)
    constexpr int KP = DK / 8, VP = DV / 8;  // 16-byte pieces per token row
    static_assert(DK % 16 == 0 && DV % 16 == 0 && 2 * TB <= NT, "prefill block shape");

    __shared__ __align__(16) uint16_t ks[TB * KR];      // keys, token-major
    __shared__ __align__(16) uint16_t kT[DK * TR];      // keys, column-major
    __shared__ __align__(16) uint16_t vT[DV * TR];      // values, column-major
    __shared__ __align__(16) float as[TB];
    __shared__ __align__(16) float bs[TB];
    __shared__ __align__(16) float Lp[NSC][kSub][4][4];       // L of each chunk: Lp[i][j % 4][j / 4] = L[i][j]
    __shared__ __align__(16) float Ts[NSC][kSub][kSub + 4];   // T = (I + L)^-1
    __shared__ __align__(16) float gs[NSC][kSub];             // g_i
    __shared__ __align__(16) float res[NSC][kSub];            // r_16i

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, q = lane >> 4;
    const int seq = blockIdx.x / p.H, h = blockIdx.x % p.H;
    const int H = p.H, L = p.L;
    const size_t tok0 = (size_t)seq * L;
    const size_t state0 = ((size_t)seq * H + h) * DV * DK;

    // S^T as accumulators: acc[c][r] = S[16 wave + n16][16 c + 4 q + r]
    f32x4 acc[KC];
    {
        const float* si = p.s_init ? p.s_init + state0 + (size_t)(16 * wave + n16) * DK + 4 * q : nullptr;
#pragma unroll
        for (int c = 0; c < KC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (si) {
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const float4 x = *reinterpret_cast<const float4*>(si + 16 * c);
                acc[c] = f32x4{x.x, x.y, x.z, x.w};
            }
        }
    }

    // staging: thread (seg, pair) moves 16-byte piece seg of the keys and values of
    // tokens 2 pair and 2 pair + 1, so the column-major copies take 4-byte writes
    static_assert(NT == (TB / 2) * KP && KP == VP, "one token pair and piece per thread");
    const int pair = tid % (TB / 2), seg = tid / (TB / 2);
    u32x4 kreg[2], vreg[2];
    float gate = 1.f;
    auto load_block = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const size_t s = tok0 + min(s0 + 2 * pair + u, L - 1);   // clamped: padding tokens are zeroed below
            kreg[u] = *reinterpret_cast<const u32x4*>(p.k + (s * H + h) * DK + seg * 8);
            vreg[u] = *reinterpret_cast<const u32x4*>(p.v + (s * H + h) * DV + seg * 8);
        }
        const int tk = tid % TB;
        const size_t s = tok0 + min(s0 + tk, L - 1);
        gate = (tid < TB ? p.alpha : p.beta)[s * H + h];           // threads 0..TB-1 alpha, TB..2TB-1 beta
    };
    auto stage_block = [&](int s0) __attribute__((always_inline)) {
        const bool in0 = s0 + 2 * pair < L, in1 = s0 + 2 * pair + 1 < L;   // padding tokens: k = v = 0
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
        const u32x4 k0 = in0 ? kreg[0] : z, k1 = in1 ? kreg[1] : z;
        const u32x4 v0 = in0 ? vreg[0] : z, v1 = in1 ? vreg[1] : z;
        *reinterpret_cast<u32x4*>(ks + (2 * pair) * KR + seg * 8) = k0;
        *reinterpret_cast<u32x4*>(ks + (2 * pair + 1) * KR + seg * 8) = k1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<uint32_t*>(kT + (seg * 8 + 2 * e) * TR + 2 * pair) = (k0[e] & 0xffffu) | (k1[e] << 16);
            *reinterpret_cast<uint32_t*>(kT + (seg * 8 + 2 * e + 1) * TR + 2 * pair) = (k0[e] >> 16) | (k1[e] & 0xffff0000u);
            *reinterpret_cast<uint32_t*>(vT + (seg * 8 + 2 * e) * TR + 2 * pair) = (v0[e] & 0xffffu) | (v1[e] << 16);
            *reinterpret_cast<uint32_t*>(vT + (seg * 8 + 2 * e + 1) * TR + 2 * pair) = (v0[e] >> 16) | (v1[e] & 0xffff0000u);
        }
        const int tk = tid % TB;
        if (tid < TB) as[tk] = s0 + tk < L ? gate : 1.f;           // padding tokens: alpha = 1, beta = 0
        else if (tid < 2 * TB) bs[tk] = s0 + tk < L ? gate : 0.f;
    };

    const int nblk = (L + TB - 1) / TB;
    if (nblk > 0) load_block(0);
    for (int blk = 0; blk < nblk; ++blk) {
        const int s0 = blk * TB;
        stage_block(s0);
        __syncthreads();
        const int nsub = min(NSC, (L - s0 + kSub - 1) / kSub);

        // ---- per chunk, state-independent: L, T = (I + L)^-1, g, r_16. ----
        for (int sc = wave; sc < nsub; sc += NW) {
            const uint16_t* kr8 = ks + (sc * kSub + n16) * KR + 8 * q;
            f32x4 G = f32x4{0.f, 0.f, 0.f, 0.f};                    // G[4q + r][n16] = k_i . k_j
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const s16x8 a = *reinterpret_cast<const s16x8*>(kr8 + 32 * kk);
                G = mfma32(a, a, G);
            }
            float al[kSub], be[4];                                   // the chunk's decays (broadcast reads)
#pragma unroll
            for (int m4 = 0; m4 < kSub / 4; ++m4) {
                const float4 x = *reinterpret_cast<const float4*>(as + sc * kSub + 4 * m4);
                al[4 * m4] = x.x; al[4 * m4 + 1] = x.y; al[4 * m4 + 2] = x.z; al[4 * m4 + 3] = x.w;
            }
            {
                const float4 x = *reinterpret_cast<const float4*>(bs + sc * kSub + 4 * q);
                be[0] = x.x; be[1] = x.y; be[2] = x.z; be[3] = x.w;
            }
            // r_ij = alpha_{j+1} ... alpha_i for i = 4q + r, j = n16 (a running product over m > j)
            float rr[4] = {0.f, 0.f, 0.f, 0.f};
            {
                float run = 1.f;
#pragma unroll
                for (int m = 0; m < kSub; ++m) {
                    run *= m > n16 ? al[m] : 1.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) rr[r] = m == 4 * q + r ? run : rr[r];
                }
            }
            // L_ij = beta_i r_ij (k_i . k_j) below the diagonal, stored as Lp[i][j % 4][j / 4]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * q + r;
                Lp[sc][i][n16 & 3][n16 >> 2] = n16 < i ? be[r] * rr[r] * G[r] : 0.f;
            }
            if (lane < kSub) {                                       // g_i = alpha_1 ... alpha_i, r_16i
                float g = 1.f, re = 1.f;
#pragma unroll
                for (int m = 0; m < kSub; ++m) {
                    g *= m <= lane ? al[m] : 1.f;
                    re *= m > lane ? al[m] : 1.f;
                }
                gs[sc][lane] = g;
                res[sc][lane] = re;
            }
            // T = (I + L)^-1 by forward substitution, four lanes per column: lane = 4 j + p
            // holds T[4k + p][j] (k = 0..3) and sums its share of each row, the quad adds up
            {
                const int j = lane >> 2, pp = lane & 3;
                float tp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < kSub; ++i) {
                    const float4 lr = *reinterpret_cast<const float4*>(&Lp[sc][i][pp][0]);   // L[i][4k + pp]
                    float sum = lr.x * tp[0];
                    sum = fmaf(lr.y, tp[1], sum);
                    sum = fmaf(lr.z, tp[2], sum);
                    sum = fmaf(lr.w, tp[3], sum);
                    sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0xB1, 0xF, 0xF, true));
                    sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0x4E, 0xF, 0xF, true));
                    const float val = (i == j ? 1.f : 0.f) - sum;
                    tp[i / 4] = pp == (i & 3) ? val : tp[i / 4];
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) Ts[sc][4 * k + pp][j] = tp[k];
            }
        }
        __syncthreads();
        if (blk + 1 < nblk) load_block(s0 + TB);                    // in flight while the chunks are folded

        // ---- per chunk, in order: the state-dependent part ----
        for (int sc = 0; sc < nsub; ++sc) {
            const uint16_t* kr = ks + (sc * kSub + n16) * KR + 4 * q;
            // P[i][v] = (S k_i)[v] for i = 4q + r, v = 16 wave + n16
            f32x4 Ph = f32x4{0.f, 0.f, 0.f, 0.f}, Pl = f32x4{0.f, 0.f, 0.f, 0.f};   // even / odd column tiles
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const s16x4 a = *reinterpret_cast<const s16x4*>(kr + 16 * c);
                s16x4 bh, bl;
                split4(acc[c], bh, bl);
                if (c & 1) Pl = mfma32(twice(a), cat(bh, bl), Pl);
                else Ph = mfma32(twice(a), cat(bh, bl), Ph);
            }
            // RHS_i = beta_i (v_i - g_i S k_i)
            const uint2 vb = *reinterpret_cast<const uint2*>(vT + (16 * wave + n16) * TR + sc * kSub + 4 * q);
            const float vv[4] = {__uint_as_float(vb.x << 16), __uint_as_float(vb.x & 0xffff0000u),
                                 __uint_as_float(vb.y << 16), __uint_as_float(vb.y & 0xffff0000u)};
            const float4 bq = *reinterpret_cast<const float4*>(bs + sc * kSub + 4 * q);
            const float4 gq = *reinterpret_cast<const float4*>(&gs[sc][4 * q]);
            const float4 rq = *reinterpret_cast<const float4*>(&res[sc][4 * q]);
            const float bv[4] = {bq.x, bq.y, bq.z, bq.w}, gv[4] = {gq.x, gq.y, gq.z, gq.w};
            const float rv[4] = {rq.x, rq.y, rq.z, rq.w};
            f32x4 rhs;
#pragma unroll
            for (int r = 0; r < 4; ++r) rhs[r] = bv[r] * (vv[r] - gv[r] * (Ph[r] + Pl[r]));
            // Delta = T RHS (both float32: hi*hi + hi*lo + lo*hi)
            const float4 tr = *reinterpret_cast<const float4*>(&Ts[sc][n16][4 * q]);
            s16x4 th, tl, rh, rl;
            split4(f32x4{tr.x, tr.y, tr.z, tr.w}, th, tl);
            split4(rhs, rh, rl);
            f32x4 dl = mfma32(twice(th), cat(rh, rl), f32x4{0.f, 0.f, 0.f, 0.f});   // T_hi (R_hi + R_lo)
            dl = mfma32(cat(tl, s16x4{0, 0, 0, 0}), cat(rh, rh), dl);                 // + T_lo R_hi
            // S' = g_16 S + K^T D with D_i = r_16i delta_i
            const float g16 = gs[sc][kSub - 1];                      // decay over the whole chunk
            f32x4 dd;
#pragma unroll
            for (int r = 0; r < 4; ++r) dd[r] = dl[r] * rv[r];
            s16x4 dh, dlo;
            split4(dd, dh, dlo);
            const uint16_t* kc = kT + n16 * TR + sc * kSub + 4 * q;
#pragma unroll
            for (int t = 0; t < KC; ++t) {
                const s16x4 a = *reinterpret_cast<const s16x4*>(kc + 16 * t * TR);
                acc[t] = mfma32(twice(a), cat(dh, dlo), acc[t] * g16);
            }
        }
        __syncthreads();                                            // LDS is restaged next
    }

    const int row = 16 * wave + n16;
    if (!PLANES) {
#pragma unroll
        for (int c = 0; c < KC; ++c)
            *reinterpret_cast<float4*>(p.s_out + state0 + (size_t)row * DK + 16 * c + 4 * q) =
                make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
    } else {
        // fragment f = (w*KS + kk)*64 + lane' holds S[16w + lane'%16][32kk + 8(lane'/16) + 0..7]
        constexpr int KS = DK / 32;
        uint16_t* pl = p.planes + ((size_t)p.slot[seq] * H + h) * 2 * DV * DK;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const int col = 16 * c + 4 * q;                       // four consecutive columns of this row
            const int kk = col / 32, ln = n16 + 16 * ((col % 32) / 8), e0 = col % 8;
            const size_t f = ((size_t)wave * KS + kk) * 64 + ln;
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = f32_to_bf16_rne(acc[c][e]);
                lo[e] = f32_to_bf16_rne(acc[c][e] - __uint_as_float(hi[e] << 16));
            }
            *reinterpret_cast<uint2*>(pl + f * 8 + e0) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
            *reinterpret_cast<uint2*>(pl + DV * DK + f * 8 + e0) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
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
