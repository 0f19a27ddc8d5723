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
// Chunks are taken in pairs (a, b): over 32 tokens the system is block lower
// triangular, so with T = (I + L)^-1 of each chunk
//   Delta_a = T_a RHS_a,
//   Delta_b = T_b (RHS_b - diag(beta_b g_b) C (r_16a . Delta_a)),  C_ij = k_(b,i) . k_(a,j),
// where RHS_b uses the decay from the pair's start (g_a16 g_b,i), and
//   S'' = g_a16 g_b16 S + sum_(j in a) g_b16 r_16j delta_j k_j^T + sum_(j in b) r_16j delta_j k_j^T.
// T and C depend only on keys and gates, so they are formed for the whole
// 64-token block before the state-dependent part runs. Per pair that part is a
// few small products on the matrix cores: P = K S^T for both chunks from one
// bf16 split of S, the two solves and the coupling, and the state update, with
// the state held as float32 accumulators of S^T (wave w owns columns
// [16w, 16w+16) of S^T, i.e. rows of S) and every float32 operand split into
// bf16 hi + lo (keys are exact in bf16). The accumulator layout of one product
// is the operand layout of the next, so nothing is reshuffled between them; the
// keys are staged in an order that lets one 16-byte LDS read supply an operand
// spanning two 16-wide tiles (or both chunks of a pair). A prompt folded in two
// calls is bit-identical to one call when the first part is a whole number of
// 32-token pairs (a trailing chunk of padding tokens is an exact no-op).
#include "onela_internal.h"

namespace onela {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 16;        // tokens per chunk (one 16x16 MFMA tile)
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

// LDS written by some lanes of a wave and then read by others of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Position of element x (0..31) of a 32-element block in the staged copies: x =
// 16 h + 4 u + e goes to 8 u + 4 h + e, so that the four values a lane group u
// takes from the first 16 and the four it takes from the second 16 sit in one
// 16-byte piece (one LDS read gives an MFMA operand spanning two 16-wide tiles).
__host__ __device__ constexpr int pair_pos(int x) { return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3); }

template <int DK, int DV, bool PLANES>
__global__ __launch_bounds__(prefill_threads<DV>(), DV >= 128 ? 4 : 1) void prefill_kernel(const PrefillParams p) {
    constexpr int NW = DV / 16;              // waves; wave w owns state rows [16w, 16w+16)
    constexpr int NT = 64 * NW;
    constexpr int KC = DK / 16;              // 16-wide column tiles of the state
    constexpr int TB = kTokBlock, NSC = kSubPerBlock, NSP = NSC / 2;
    constexpr int KR = DK + 8;               // LDS row of a token's key (bf16)
    constexpr int TR = TB + 8;               // LDS row of a key / value column over the block's tokens (bf16)
    constexpr int KP = DK / 8, VP = DV / 8;  // 16-byte pieces per token row
    static_assert(DK % 32 == 0 && DV % 16 == 0 && 2 * TB <= NT && NSC % 2 == 0, "prefill block shape");

    __shared__ __align__(16) uint16_t ks[TB * KR];      // keys, token-major, elements in pair_pos order
    __shared__ __align__(16) uint16_t kT[DK * TR];      // keys, column-major, tokens in pair_pos order
    __shared__ __align__(16) uint16_t vT[DV * TR];      // values, column-major
    __shared__ __align__(16) float as[TB];
    __shared__ __align__(16) float bs[TB];
    constexpr int LRC = kSub * kSub + 4;     // floats per chunk of Lr
    __shared__ __align__(16) float Lr[NSC * LRC];             // L of each chunk, row-major
    __shared__ __align__(16) float Ts[NSC][kSub][kSub + 4];   // T = (I + L)^-1
    __shared__ __align__(16) float Cs[NSP][kSub][kSub + 4];   // k_i . k_j, i in the second chunk of a pair, j in the first
    __shared__ __align__(16) float gs[NSC][kSub];             // g_i
    __shared__ __align__(16) float res[NSC][kSub];            // r_16i
    // MFMA A-operands in bf16: [m][0][u][i] = hi of row i, columns 4u..4u+3, twice;
    // [m][1][u][i] = lo, then zeros (a wave's read of one half is 1 KB in lane order)
    __shared__ __align__(16) s16x8 Top[NSC][2][4][kSub];      // T of each chunk
    __shared__ __align__(16) s16x8 Cop[NSP][2][4][kSub];      // C of each pair

    const int tid = threadIdx.x, wave = tid >> 6;
    const int seq = blockIdx.x / p.H, h = blockIdx.x % p.H;
    const int H = p.H, L = p.L;
    const size_t tok0 = (size_t)seq * L;
    const size_t state0 = ((size_t)seq * H + h) * DV * DK;

    // S^T as accumulators: acc[c][r] = S[16 wave + n16][16 c + 4 q + r]
    f32x4 acc[KC];
    {
        const int n16 = tid & 15, q = (tid & 63) >> 4;
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
        // (the initial state is complete before the block loop: otherwise the wait for it,
        // placed inside the loop, would also wait for the next block's loads every time)
#pragma unroll
        for (int c = 0; c < KC; ++c) asm volatile("" ::"v"(acc[c]));
    }

    // staging: thread (seg, pair) moves 16-byte piece seg of the keys and values of
    // tokens 2 pair and 2 pair + 1, so the column-major copies take 4-byte writes
    // (every per-lane index below comes from the thread id passed in, an opaque copy
    // made per block: values derived from it are not hoisted out of the block loop,
    // where at 128 registers per lane they would be spilled)
    static_assert(NT == (TB / 2) * KP && KP == VP, "one token pair and piece per thread");
    u32x4 kreg[2], vreg[2];
    float gate = 1.f;
    const float* const alpha_in = p.alpha;
    const float* const beta_in = p.beta;
    auto load_block = [&](int s0, int tid) __attribute__((always_inline)) {
        const int pair = tid % (TB / 2), seg = tid / (TB / 2);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const size_t s = tok0 + min(s0 + 2 * pair + u, L - 1);   // (clamped: padding repeats token L-1)
            kreg[u] = *reinterpret_cast<const u32x4*>(p.k + (s * H + h) * DK + seg * 8);
            vreg[u] = *reinterpret_cast<const u32x4*>(p.v + (s * H + h) * DV + seg * 8);
        }
        const int tk = tid % TB;
        const size_t s = tok0 + min(s0 + tk, L - 1);
        gate = (tid < TB ? alpha_in : beta_in)[s * H + h];         // threads 0..TB-1 alpha, TB..2TB-1 beta
    };
    auto stage_block = [&](int s0, int tid) __attribute__((always_inline)) {
        const int pair = tid % (TB / 2), seg = tid / (TB / 2);
        // padding tokens (past L) carry the last token's k and v: with alpha = 1 and beta = 0
        // every term they enter is multiplied by their beta or their delta, both 0
        const u32x4 k0 = kreg[0], k1 = kreg[1], v0 = vreg[0], v1 = vreg[1];
        // elements 8 seg .. 8 seg + 7 are two groups of four, each contiguous in pair_pos order
        const int e0 = pair_pos(8 * seg), e1 = pair_pos(8 * seg + 4);
        *reinterpret_cast<uint2*>(ks + (2 * pair) * KR + e0) = make_uint2(k0[0], k0[1]);
        *reinterpret_cast<uint2*>(ks + (2 * pair) * KR + e1) = make_uint2(k0[2], k0[3]);
        *reinterpret_cast<uint2*>(ks + (2 * pair + 1) * KR + e0) = make_uint2(k1[0], k1[1]);
        *reinterpret_cast<uint2*>(ks + (2 * pair + 1) * KR + e1) = make_uint2(k1[2], k1[3]);
        const int tpos = pair_pos(2 * pair);                       // tokens 2 pair, 2 pair + 1 stay adjacent
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // (one byte permute per word: low halves, then high halves)
            *reinterpret_cast<uint32_t*>(kT + (seg * 8 + 2 * e) * TR + tpos) = __builtin_amdgcn_perm(k1[e], k0[e], 0x05040100u);
            *reinterpret_cast<uint32_t*>(kT + (seg * 8 + 2 * e + 1) * TR + tpos) = __builtin_amdgcn_perm(k1[e], k0[e], 0x07060302u);
            *reinterpret_cast<uint32_t*>(vT + (seg * 8 + 2 * e) * TR + 2 * pair) = __builtin_amdgcn_perm(v1[e], v0[e], 0x05040100u);
            *reinterpret_cast<uint32_t*>(vT + (seg * 8 + 2 * e + 1) * TR + 2 * pair) = __builtin_amdgcn_perm(v1[e], v0[e], 0x07060302u);
        }
        const int tk = tid % TB;
        if (tid < TB) as[tk] = s0 + tk < L ? gate : 1.f;           // padding tokens: alpha = 1, beta = 0
        else if (tid < 2 * TB) bs[tk] = s0 + tk < L ? gate : 0.f;
    };

    // row i = lane % 16, columns 4u..4u+3 (u = lane / 16) of a 16 x 16 float32 matrix in LDS
    // (rows of kSub + 4) as the bf16 A-operand records {hi twice}, {lo, zeros}
    auto write_operand = [&](const float* m, s16x8 (*dst)[4][kSub], int lane) __attribute__((always_inline)) {
        const int i = lane & 15, u = lane >> 4;
        const float4 x = *reinterpret_cast<const float4*>(m + i * (kSub + 4) + 4 * u);
        s16x4 hi, lo;
        split4(f32x4{x.x, x.y, x.z, x.w}, hi, lo);
        dst[0][u][i] = twice(hi);
        dst[1][u][i] = cat(lo, s16x4{0, 0, 0, 0});
    };

    const int nblk = (L + TB - 1) / TB;
    if (nblk > 0) load_block(0, tid);
    for (int blk = 0; blk < nblk; ++blk) {
        const int s0 = blk * TB;
        int tid_l = tid;
        asm volatile("" : "+v"(tid_l));
        const int lane = tid_l & 63, n16 = lane & 15, q = lane >> 4;
        stage_block(s0, tid_l);
        __syncthreads();
        // chunk pairs holding prompt tokens (a trailing chunk of padding is an exact no-op)
        const int npair = min(NSP, (L - s0 + 2 * kSub - 1) / (2 * kSub));

        // ---- state-independent part, one task per wave (all chunks of the block are staged,
        // padding included, so every chunk is formed). Tasks 0 .. NSC-1: a chunk's L, g, r_16
        // and T = (I + L)^-1; tasks NSC ..: the key products C between the two chunks of a
        // pair. T and C leave as bf16 hi/lo MFMA A-operands (Top, Cop) ----
        for (int task = wave; task < NSC + NSP; task += NW) {
            if (task >= NSC) {
                // C_ij = k_i . k_j, i in chunk b, j in chunk a of pair sp
                const int sp = task - NSC, a = 2 * sp, b = a + 1;
                const uint16_t* kb = ks + (b * kSub + n16) * KR + 8 * q;
                const uint16_t* ka = ks + (a * kSub + n16) * KR + 8 * q;
                f32x4 C = f32x4{0.f, 0.f, 0.f, 0.f};                // C[4q + e][n16]
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    C = mfma32(*reinterpret_cast<const s16x8*>(kb + 32 * kk), *reinterpret_cast<const s16x8*>(ka + 32 * kk), C);
#pragma unroll
                for (int e = 0; e < 4; ++e) Cs[sp][4 * q + e][n16] = C[e];
                wave_lds_sync();
                write_operand(&Cs[sp][0][0], Cop[sp], lane);
                continue;
            }
            const int sc = task;
            const uint16_t* kr8 = ks + (sc * kSub + n16) * KR + 8 * q;
            f32x4 G = f32x4{0.f, 0.f, 0.f, 0.f};                    // G[4q + e][n16] = k_i . k_j
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const s16x8 a = *reinterpret_cast<const s16x8*>(kr8 + 32 * kk);
                G = mfma32(a, a, G);
            }
            // r_ij = alpha_{j+1} ... alpha_i for i = 4q + e, j = n16: the product of
            // a_m = (m > j ? alpha_m : 1) over m <= i, taken within the lane group
            // (m = 4q .. 4q+3) and then across the groups below (same column)
            const float4 a4 = *reinterpret_cast<const float4*>(as + sc * kSub + 4 * q);
            const float4 b4 = *reinterpret_cast<const float4*>(bs + sc * kSub + 4 * q);
            const float av[4] = {a4.x, a4.y, a4.z, a4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
            float rr[4], run = 1.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                run *= 4 * q + e > n16 ? av[e] : 1.f;
                rr[e] = run;
            }
            float x = run;                                          // inclusive scan of the group totals
            float y = __shfl_up(x, 16, 64);
            x = q >= 1 ? x * y : x;
            y = __shfl_up(x, 32, 64);
            x = q >= 2 ? x * y : x;
            y = __shfl_up(x, 16, 64);                               // exclusive: groups below this one
            const float below = q >= 1 ? y : 1.f;
            float* lrow = Lr + sc * LRC + 4 * q * kSub + n16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rr[e] *= below;
                lrow[e * kSub] = n16 < 4 * q + e ? bv[e] * rr[e] * G[e] : 0.f;   // L_ij, j < i
            }
            if (n16 == 0) {                                         // g_i = alpha_1 r_i1 (1-based)
                const float a0 = as[sc * kSub];
#pragma unroll
                for (int e = 0; e < 4; ++e) gs[sc][4 * q + e] = a0 * rr[e];
            }
            if (q == 3) res[sc][n16] = rr[3];                       // r_16j = r_(16, j)
            wave_lds_sync();
            // T by forward substitution, lane j < 16 holding column j
            if (lane < kSub) {
                const float* L0 = Lr + sc * LRC;
                float t[kSub];
#pragma unroll
                for (int i = 0; i < kSub; ++i) {
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int m = 0; m + 1 < i; m += 2) {
                        s0 = fmaf(L0[i * kSub + m], t[m], s0);
                        s1 = fmaf(L0[i * kSub + m + 1], t[m + 1], s1);
                    }
                    if (i & 1) s0 = fmaf(L0[i * kSub + i - 1], t[i - 1], s0);
                    t[i] = (i == lane ? 1.f : 0.f) - (s0 + s1);
                }
#pragma unroll
                for (int i = 0; i < kSub; ++i) Ts[sc][i][lane] = t[i];
            }
            wave_lds_sync();
            write_operand(&Ts[sc][0][0], Top[sc], lane);
        }
        __syncthreads();
        if (blk + 1 < nblk) load_block(s0 + TB, tid_l);                    // in flight while the chunks are folded

        // ---- per chunk pair (a, b), in order: the state-dependent part.
        // P = K S^T for both chunks from one split of S; Delta_a = T_a RHS_a;
        // Delta_b = T_b (RHS_b - diag(beta_b g_b) C (r_16a . Delta_a)) (the 32-token system is
        // block lower triangular); S^T <- g_a16 g_b16 S^T + K_a^T D_a + K_b^T D_b with
        // D_a = g_b16 r_16a . Delta_a, D_b = r_16b . Delta_b ----
        for (int sp = 0; sp < npair; ++sp) {
            const int a = 2 * sp, b = a + 1;
            // The vector ALUs are the bottleneck here and the issue arbiter favours older
            // waves, so the upper half of the workgroup would fall behind and the lower
            // half wait for it at the block's barrier: the halves take turns at the higher
            // priority, one chunk pair each.
            if ((wave >= NW / 2) != (sp & 1)) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            const uint16_t* kra = ks + (a * kSub + n16) * KR + 8 * q;
            const uint16_t* krb = kra + kSub * KR;
            // P[i][v] = (S k_i)[v] for i = 4q + r, v = 16 wave + n16; two chains per chunk (hi, lo)
            f32x4 Xa = f32x4{0.f, 0.f, 0.f, 0.f}, Ya = Xa, Xb = Xa, Yb = Xa;
#pragma unroll
            for (int cp = 0; cp < KC / 2; ++cp) {
                s16x4 h0, l0, h1, l1;
                split4(acc[2 * cp], h0, l0);
                split4(acc[2 * cp + 1], h1, l1);
                const s16x8 bh = cat(h0, h1), bl = cat(l0, l1);
                const s16x8 ka8 = *reinterpret_cast<const s16x8*>(kra + 32 * cp);
                const s16x8 kb8 = *reinterpret_cast<const s16x8*>(krb + 32 * cp);
                Xa = mfma32(ka8, bh, Xa);
                Ya = mfma32(ka8, bl, Ya);
                Xb = mfma32(kb8, bh, Xb);
                Yb = mfma32(kb8, bl, Yb);
            }
            const float4 gaq = *reinterpret_cast<const float4*>(&gs[a][4 * q]);
            const float4 gbq = *reinterpret_cast<const float4*>(&gs[b][4 * q]);
            const float4 raq = *reinterpret_cast<const float4*>(&res[a][4 * q]);
            const float4 rbq = *reinterpret_cast<const float4*>(&res[b][4 * q]);
            const float4 baq = *reinterpret_cast<const float4*>(bs + a * kSub + 4 * q);
            const float4 bbq = *reinterpret_cast<const float4*>(bs + b * kSub + 4 * q);
            const float ga16 = gs[a][kSub - 1], gb16 = gs[b][kSub - 1];
            const uint2 vab = *reinterpret_cast<const uint2*>(vT + (16 * wave + n16) * TR + a * kSub + 4 * q);
            const uint2 vbb = *reinterpret_cast<const uint2*>(vT + (16 * wave + n16) * TR + b * kSub + 4 * q);
            // RHS_a,i = beta_i (v_i - g_i S k_i)
            const f32x4 rhs_a = f32x4{baq.x * (__uint_as_float(vab.x << 16) - gaq.x * (Xa[0] + Ya[0])),
                                      baq.y * (__uint_as_float(vab.x & 0xffff0000u) - gaq.y * (Xa[1] + Ya[1])),
                                      baq.z * (__uint_as_float(vab.y << 16) - gaq.z * (Xa[2] + Ya[2])),
                                      baq.w * (__uint_as_float(vab.y & 0xffff0000u) - gaq.w * (Xa[3] + Ya[3]))};
            // RHS_b,i = beta_i (v_i - g_a16 g_i S k_i), before the coupling to chunk a
            f32x4 rhs_b = f32x4{bbq.x * (__uint_as_float(vbb.x << 16) - ga16 * gbq.x * (Xb[0] + Yb[0])),
                                bbq.y * (__uint_as_float(vbb.x & 0xffff0000u) - ga16 * gbq.y * (Xb[1] + Yb[1])),
                                bbq.z * (__uint_as_float(vbb.y << 16) - ga16 * gbq.z * (Xb[2] + Yb[2])),
                                bbq.w * (__uint_as_float(vbb.y & 0xffff0000u) - ga16 * gbq.w * (Xb[3] + Yb[3]))};
            // Delta_a = T_a RHS_a (float32 both: hi*hi + hi*lo + lo*hi)
            s16x4 h, l;
            split4(rhs_a, h, l);
            s16x8 bop = cat(h, l);
            f32x4 da = mfma32(Top[a][0][q][n16], bop, f32x4{0.f, 0.f, 0.f, 0.f});
            da = mfma32(Top[a][1][q][n16], bop, da);
            // RHS_b,i -= beta_i g_i sum_j C_ij r_16j delta_j, then Delta_b = T_b RHS_b
            const f32x4 xa = f32x4{da[0] * raq.x, da[1] * raq.y, da[2] * raq.z, da[3] * raq.w};
            split4(xa, h, l);
            bop = cat(h, l);
            f32x4 cx = mfma32(Cop[sp][0][q][n16], bop, f32x4{0.f, 0.f, 0.f, 0.f});
            cx = mfma32(Cop[sp][1][q][n16], bop, cx);
            rhs_b[0] = fmaf(-bbq.x * gbq.x, cx[0], rhs_b[0]);
            rhs_b[1] = fmaf(-bbq.y * gbq.y, cx[1], rhs_b[1]);
            rhs_b[2] = fmaf(-bbq.z * gbq.z, cx[2], rhs_b[2]);
            rhs_b[3] = fmaf(-bbq.w * gbq.w, cx[3], rhs_b[3]);
            split4(rhs_b, h, l);
            bop = cat(h, l);
            f32x4 db = mfma32(Top[b][0][q][n16], bop, f32x4{0.f, 0.f, 0.f, 0.f});
            db = mfma32(Top[b][1][q][n16], bop, db);
            // the state update: D_a, D_b as bf16 hi + lo against the keys of both chunks
            s16x4 dha, dla, dhb, dlb;
            split4(xa * gb16, dha, dla);
            split4(f32x4{db[0] * rbq.x, db[1] * rbq.y, db[2] * rbq.z, db[3] * rbq.w}, dhb, dlb);
            const s16x8 uh = cat(dha, dhb), ul = cat(dla, dlb);
            const float g32 = ga16 * gb16;                           // decay over the whole pair
            const uint16_t* kc = kT + n16 * TR + a * kSub + 8 * q;
#pragma unroll
            for (int t = 0; t < KC; ++t) {
                const s16x8 kt8 = *reinterpret_cast<const s16x8*>(kc + 16 * t * TR);
                acc[t] = mfma32(kt8, uh, acc[t] * g32);
                acc[t] = mfma32(kt8, ul, acc[t]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();                                            // LDS is restaged next
    }

    const int n16 = tid & 15, q = (tid & 63) >> 4;
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
