// gfx950 kernels of the OneLA large-beam GDN decode step.
//
// One launch per decode step of one GDN layer (OneLA abstract: a fused GPU
// kernel reuses the shared state across beams). A workgroup owns one
// (request, head) pair and a range of beams. It first derives the request's
// beam processing order for this step (beams grouped by ancestry, so that a
// chunk gathers records other chunks mostly do not need), then walks its
// range in that order in chunks of kChunk beams. For each chunk it
//   A. stages k_t and q_t of the chunk's beams in LDS and builds each beam's
//      ancestry row from its parent's row (record ids only; OneLA abstract:
//      records are never moved or copied);
//   B. computes, per beam and ancestral record j, the dot products k_j . k_t
//      and k_j . q_t, the only way the replay touches x (OneLA review,
//      "Scope & Claims": the recurrence right-multiplied by q_t and k_t,
//      paper Eq. 3), plus k_t . q_t;
//   C. projects the shared state once for all 2*kChunk vectors,
//      P = S0 [k_t q_t], on the matrix cores (split-bf16: S0 = hi + lo);
//   D. completes the replay in the MFMA accumulator registers, forms
//      delta_t = beta (v - alpha y_k) and o_t = alpha y_q + (k_t . q_t) delta_t
//      (= S_t q_t), and appends (alpha_t, delta_t, k_t) at the beam's
//      processing position, so a chunk's records are adjacent.
//
// Wave w of the workgroup owns rows [16w, 16w+16) of d_v: its slice of S0
// stays in registers as MFMA A-fragments for the whole beam loop, and every
// step after the projection is row-separable, so no wave needs another
// wave's rows. After the beam loop
// (one head per request, unless the index belongs to another layer's
// context) the next step's ancestry rows are written in beam-index order.
//
// Variants: in graph mode each request's step index comes from device
// memory and the last workgroup of the request advances it; the FUSED
// instantiation takes raw projections (per-head L2 normalisation of q and k,
// the decay and write-strength gates) and writes o as bf16; a request at its
// first step has no ancestral records and runs a body without the gathers.
#include "onela_internal.h"

namespace onela {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWave = 16;     // d_v rows per wave (one 16x16x32 MFMA tile row block)
constexpr int kAncBatch = 8;         // ancestry-row entries copied per round of loads

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// sum of the 8 bf16 products of a and b, plus acc, in fp32 (packed dot2)
__device__ __forceinline__ float dot8(uint4 a, uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
    return acc;
}

// Workgroup barrier that orders LDS only. Inside one step launch no thread
// reads global memory another thread of the launch wrote (records of this
// step are appended at ids no one reads before the next launch), so the
// barriers need not wait for outstanding global stores.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// S0 (float32, row-major [H][DV][DK]) -> two bf16 planes hi, lo with
// hi = rne(S0), lo = rne(S0 - hi), stored in the order the step kernel loads
// its MFMA A-fragments: fragment f = (w*KS + kk)*64 + lane holds the 8 values
// S0[16w + lane%16][32kk + 8*(lane/16) + 0..7].
template <int DK, int DV>
__global__ __launch_bounds__(256) void init_s0_kernel(const float* __restrict__ S0,
                                                      uint16_t* __restrict__ planes, int H) {
    constexpr int KS = DK / 32;
    constexpr int NFRAG = DV * DK / 8;
    const int f = blockIdx.x * 256 + threadIdx.x;
    if (f >= H * NFRAG) return;
    const int h = f / NFRAG, fi = f % NFRAG;
    const int lane = fi & 63, wk = fi >> 6;
    const int w = wk / KS, kk = wk % KS;
    const int m = kRowsPerWave * w + (lane & 15);
    const int kb = 32 * kk + 8 * (lane >> 4);
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
template <int DV>
__host__ __device__ constexpr int step_threads() { return 64 * (DV / kRowsPerWave); }

// Input-side fusion: a layer's raw gate projections to the step's decay and
// write strength, alpha = exp(-exp(A_log) softplus(a + dt_bias)) and
// beta = sigmoid(b) (the usual gated DeltaNet parametrisation; the pages do
// not describe it).
__device__ __forceinline__ float gate_alpha(float a_raw, float neg_A, float dt_bias) {
    const float x = a_raw + dt_bias;
    const float softplus = x > 20.f ? x : log1pf(expf(x));
    return expf(neg_A * softplus);
}

__device__ __forceinline__ float gate_beta(float b_raw) { return 1.f / (1.f + expf(-b_raw)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// FUSED: q, k arrive as raw projections and are L2-normalised per head in
// phase A (float32, rounded to bf16 before any use, so records hold the keys
// the step used); alpha and beta arrive raw; o leaves as bf16.
// HIST = false: the workgroup's request takes its first step (no ancestral
// records), so no record is gathered. With nothing to gather, its chunks are
// half as long: shorter staging and compute phases interleave better between
// the workgroups that share a CU.
// HCH: beams per chunk of the general body, kChunk, or kChunk / 2 for
// launches too small to fill the GPU (more workgroups, each with fewer beams).
template <int DK, int DV, bool FUSED, bool HIST, int HCH>
__device__ __forceinline__ void step_body(const StepParams& p) {
    constexpr int CH = HIST ? HCH : kChunk / 2;
    constexpr int NW = DV / kRowsPerWave;
    constexpr int NT = 64 * NW;
    constexpr int KS = DK / 32;        // MFMA k-steps
    constexpr int NG = CH / 32;        // 32-beam groups per chunk
    constexpr int XS = DK + 16;        // padded LDS row (bf16 elements): B-fragment reads free of bank conflicts
    constexpr int MT = CH / 16;        // 16-beam tiles per chunk
    constexpr int TPQ = NT / kChunk;   // threads per beam for k_t . q_t (the same split at both chunk
    constexpr int EQ = DK / TPQ;       // lengths, so both instantiations round it alike); elements per thread
    static_assert(TPQ >= 1 && EQ % 8 == 0, "k_t . q_t split");
    static_assert((2 * CH * (DK / 8)) % NT == 0 && (CH * (DV / 8)) % NT == 0, "whole stream loads per thread");
    constexpr int DBD = 2;             // depths whose delta gathers are in flight together
    constexpr int UPP = 2;             // dot-product units per wave whose key gathers are in flight together
    constexpr int VS = DV + 16;        // padded LDS row of v (bf16 elements)
    static_assert(DV % kRowsPerWave == 0 && DK % 32 == 0, "tile shape");

    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int MS = p.T_max > 1 ? p.T_max - 1 : 1;                  // ancestry depth capacity
    float4* coef_s = reinterpret_cast<float4*>(lds_raw);            // [MS][CH] {k_j.k_t, k_j.q_t, alpha_j, rid}
    uint16_t* xs = reinterpret_cast<uint16_t*>(coef_s + CH * MS);   // [2*CH][XS]: k rows then q rows
    uint16_t* vs = xs + 2 * CH * XS;                                // [CH][VS]: v rows
    int* anc_s = reinterpret_cast<int*>(vs + CH * VS);              // [MS][CH] record ids, oldest first
    float* kq_s = reinterpret_cast<float*>(anc_s + CH * MS);        // [CH]: k_t . q_t
    float* at_s = kq_s + CH;                                        // [CH]: alpha_t
    float* bt_s = at_s + CH;                                        // [CH]: beta_t
    const int Wp = (p.W + 3) & ~3;                                   // W rounded up to whole int4s
    int* ord_s = reinterpret_cast<int*>(bt_s + CH);                 // [Wp] beam at each position of this step's order
    int* posp_s = ord_s + Wp;                                       // [Wp] position of each beam in step t-1's order
    int* ck_s = reinterpret_cast<int*>(xs);                         // before the beam loop: sort keys or sort scratch
    static_assert(!HIST || (2 * CH * XS + CH * VS) * 2 >= kOrderMax * 4, "sort keys fit in the k/q/v staging area");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Workgroups are dealt to the 8 XCDs round-robin; renumber them so that
    // the beam splits of one (request, head), and the heads of one request,
    // land on one XCD and share its L2.
    int L = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) L = (L & 7) * (nblk >> 3) + (L >> 3);
    const int split = L % p.n_splits;
    const int pair = L / p.n_splits;
    const int ri = pair / p.H;
    const int h = pair % p.H;
    const int slot = p.slot[ri];
    int t = p.t[ri], epoch = p.epoch[ri];
    if (p.dev_steps) {                            // graph mode: the counters live on the device
        t = p.dev_steps[slot] + 1;
        epoch = p.dev_epoch[slot];
    }
    // The previous step's beam order and this step's parents are loaded
    // first, so that the ordering below overlaps the S0 loads. The order is
    // read at both step parities: in graph mode the step index is not known
    // before its counter arrives. (Indices clamped into the arrays; the
    // values go unused at t = 1.)
    constexpr int OU = (kOrderMax + NT - 1) / NT;
    int po0[OU], po1[OU], pa[OU];
    {
        const int* order0 = p.order + (size_t)slot * p.W;
        const int* order1 = p.order + ((size_t)p.max_requests + slot) * p.W;
        const int* prow = p.parent ? p.parent + (size_t)ri * p.W : order0;
#pragma unroll
        for (int u = 0; u < OU; ++u) {
            const int i = min(tid + u * NT, p.W - 1);
            po0[u] = order0[i];
            po1[u] = order1[i];
            pa[u] = prow[i];
        }
    }
    // Graph mode: the last workgroup of a request to finish advances its step
    // counter. Every wave reads the counter before its first barrier, and
    // thread 0 counts its workgroup only after the last one, so no workgroup
    // of the launch can see the advanced value.
    auto count_done = [&]() __attribute__((always_inline)) {
        if (p.dev_steps && threadIdx.x == 0) {
            const int before = atomicAdd(&p.done[slot], 1);
            if (before == p.H * p.n_splits - 1) {
                p.done[slot] = 0;
                if (t <= p.T_max) p.dev_steps[slot] = t;
            }
        }
    };
    if (t > p.T_max) {                            // (graph mode) no record slot left: report, write nothing
        if (threadIdx.x == 0) p.err_cap[slot] = epoch;
        count_done();
        return;
    }
    const int H = p.H, W = p.W;
    const int depth = HIST ? t - 1 : 0;           // ancestral records per beam
    const int b_begin = split * p.beams_per_block;
    const int b_end = min(W, b_begin + p.beams_per_block);
    if (b_begin >= b_end) {
        count_done();
        return;
    }

    // Uniform 64-bit bases of this (request, head); every per-lane offset from
    // them is a 32-bit int (the host rejects shapes where that could overflow).
    const size_t pair_id = (size_t)slot * H + h;
    const size_t rec0 = pair_id * (size_t)p.T_max * W;            // record 0 of this (request, head)
    const size_t in0 = (size_t)ri * W * H + h;                     // input row of (beam 0, head h)
    const int HK = H * DK, HV = H * DV;                            // input row strides between beams
    const uint16_t* kin = p.k + in0 * DK;
    const uint16_t* qin = p.q + in0 * DK;
    const uint16_t* vin = p.v + in0 * DV;
    const float* ain = p.alpha + in0;
    const float* bin = p.beta + in0;
    float* oout = FUSED ? nullptr : p.o + in0 * DV;
    uint16_t* oout16 = FUSED ? p.o_bf16 + in0 * DV : nullptr;
    // (uniform values, kept in scalar registers)
    const float neg_A = FUSED ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(-expf(p.A_log[h])))) : 0.f;
    const float dtb = FUSED ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(p.dt_bias[h]))) : 0.f;
    float* dout = p.delta_out ? p.delta_out + in0 * DV : nullptr;
    const int* parin = depth > 0 ? p.parent + (size_t)ri * W : nullptr;
    // Record r of step j is the one written by the beam at position r - jW of
    // step j's processing order, so the beams of a chunk append adjacent
    // records and a chunk's ancestors of one depth are nearly adjacent too.
    float* ralpha = p.rec_alpha + rec0;                            // record r: ralpha[r]
    float* rdw = p.rec_delta + rec0 * DV + __builtin_amdgcn_readfirstlane(wave) * kRowsPerWave;   // wave's rows of record r: rdw + r*DV
    uint16_t* rkey = p.rec_k + rec0 * DK;                          // record r: rkey + r*DK
    const int* anc_prev = p.anc + ((size_t)((t - 1) & 1) * p.max_requests + slot) * (size_t)W * p.T_max;
    int* anc_next = p.anc + ((size_t)(t & 1) * p.max_requests + slot) * (size_t)W * p.T_max;
    int* ord_next = p.order + ((size_t)(t & 1) * p.max_requests + slot) * W;

    // Up to kOrderMax beams, every step has an order (the identity when not
    // sorted), kept in an LDS table: ord_s maps positions to beams, posp_s the
    // previous step's beams to their positions. The index owner sorts (when
    // the host asks for it) and writes the order; a layer sharing the index
    // reads the owner's order of this step, so every layer puts a beam's
    // record at the same position.
    const bool track = W <= kOrderMax;
    const bool sharer = !p.write_index;
    const bool ordered = track && !sharer && p.order_beams && depth > 0;
    constexpr int kRankMaxW = 256;   // widest beam set ranked by comparisons; wider ones are radix-sorted
    __builtin_amdgcn_sched_barrier(0);

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

    // Beams are processed in an order that groups the beam tree: at step t a
    // beam's sort key is its parent's position in step t-1's order (ties by
    // beam index), so siblings are adjacent and beams sharing older ancestors
    // are near each other; a chunk then gathers mostly records that no other
    // chunk needs. Each beam's arithmetic is independent of the order. Every
    // workgroup of the owner derives the same order (a deterministic rank),
    // and one of them writes it, for the next step and for the sharing layers
    // of this one. Wider beam sets than kOrderMax keep the natural order.
    if (track) {
        if (depth == 0) {
            for (int i = tid; i < W; i += NT) ord_s[i] = i;
        } else {
#pragma unroll
            for (int u = 0; u < OU; ++u) {
                const int i = tid + u * NT;
                const int po = (depth & 1) ? po1[u] : po0[u];                 // order of step t-1
                const int pc = (depth & 1) ? po0[u] : po1[u];                 // the owner's order of step t
                if (i < W) {
                    posp_s[min((unsigned)po, (unsigned)(W - 1))] = i;         // position of each step t-1 beam
                    if (sharer) ord_s[i] = min((unsigned)pc, (unsigned)(W - 1));
                    else if (!ordered) ord_s[i] = i;
                }
            }
            lds_barrier();
            if (ordered && W <= kRankMaxW) {
#pragma unroll
                for (int u = 0; u < OU; ++u) {
                    const int i = tid + u * NT;
                    const int pb = pa[u];
                    if (i < Wp)   // unique composite keys; the padding sorts last
                        ck_s[i] = i < W ? (int)min((unsigned)posp_s[(pb < 0 || pb >= W) ? 0 : pb], (unsigned)(W - 1)) * W + i
                                        : 0x7fffffff;
                    if (i < W) ord_s[i] = i;   // (overwritten by the ranks below)
                }
                lds_barrier();
                // rank of each key among all keys: G adjacent lanes share a beam
                // and split its key range, reading four keys per LDS access
                int G = 1;
                while (G < 8 && 2 * G * W <= NT) G <<= 1;
                const int g = tid & (G - 1);
                const int nq = Wp >> 2;
                const int4* ck4 = reinterpret_cast<const int4*>(ck_s);
                for (int b0 = 0; b0 < W; b0 += NT / G) {
                    const int b = b0 + tid / G;
                    const int c = ck_s[min(b, W - 1)];
                    int r = 0;
#pragma unroll 4
                    for (int qd = g; qd < nq; qd += G) {
                        const int4 kv = ck4[qd];
                        r += (kv.x < c) + (kv.y < c) + (kv.z < c) + (kv.w < c);
                    }
                    for (int m = 1; m < G; m <<= 1) r += __shfl_xor(r, m, 64);
                    if (g == 0 && b < W) ord_s[r] = b;
                }
            } else if (ordered) {
                // Stable LSD radix sort of the beams, from index order, by the
                // parent's position in step t-1's order, RB bits a pass: the order
                // of the keys (parent position, beam index). Each entry packs the
                // parent position above the beam index. Per pass, every 64-beam
                // chunk counts its digits and ranks its beams within the chunk by
                // ballots; a scan of the counts (digit-major) gives every chunk's
                // first slot per digit, and each beam moves to its slot.
                static_assert(kOrderMax <= 1024, "beam index in 10 bits");
                constexpr int SCR = (2 * CH * XS + CH * VS) * 2;              // bytes of the staging area
                constexpr int NCHM = kOrderMax / 64;
                constexpr int RB = 2 * kOrderMax * 4 + 32 * NCHM * 4 <= SCR ? 5 : 4;
                constexpr int RD = 1 << RB;
                static_assert(2 * kOrderMax * 4 + RD * NCHM * 4 <= SCR, "sort scratch fits in the staging area");
                constexpr int CPW = (NCHM + NW - 1) / NW;                     // chunks per wave
                const int nch = (W + 63) >> 6;
                int* sqa = ck_s;                                              // [Wp] (parent position << 10) | beam
                int* sqb = sqa + Wp;                                          // [Wp]
                int* hs = sqb + Wp;                                           // [RD][nch] counts, then first slots
#pragma unroll
                for (int u = 0; u < OU; ++u) {
                    const int i = tid + u * NT;
                    const int pb = pa[u];
                    if (i < W)
                        sqa[i] = (int)(min((unsigned)posp_s[(pb < 0 || pb >= W) ? 0 : pb], (unsigned)(W - 1)) << 10) | i;
                }
                lds_barrier();
                const int nbits = W > 1 ? 32 - __clz(W - 1) : 0;
                for (int sh = 0; sh < nbits; sh += RB) {
                    int ent[CPW], dg[CPW], rk[CPW];
#pragma unroll
                    for (int k = 0; k < CPW; ++k) {
                        const int c = wave + k * NW;
                        const int i = c * 64 + lane;
                        const bool valid = c < nch && i < W;
                        ent[k] = valid ? sqa[i] : 0;
                        dg[k] = valid ? (ent[k] >> (10 + sh)) & (RD - 1) : RD;   // RD: no beam
                        rk[k] = 0;
                        if (c < nch) {                                        // (uniform in the wave)
#pragma unroll 1
                            for (int v = 0; v < RD; ++v) {
                                const unsigned long long m = __ballot(dg[k] == v);
                                if (dg[k] == v)
                                    rk[k] = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
                                if (lane == v) hs[v * nch + c] = __popcll(m);
                            }
                        }
                    }
                    lds_barrier();
                    if (wave == 0) {                                          // exclusive scan, digit-major
                        constexpr int EM = (RD * NCHM + 63) / 64;
                        const int S = RD * nch;
                        int loc[EM], sum = 0;
#pragma unroll
                        for (int e = 0; e < EM; ++e) {
                            const int j = lane * EM + e;
                            loc[e] = j < S ? hs[j] : 0;
                            sum += loc[e];
                        }
                        int x = sum;
#pragma unroll
                        for (int o = 1; o < 64; o <<= 1) {
                            const int y = __shfl_up(x, o, 64);
                            if (lane >= o) x += y;
                        }
                        int run = x - sum;
#pragma unroll
                        for (int e = 0; e < EM; ++e) {
                            const int j = lane * EM + e;
                            if (j < S) hs[j] = run;
                            run += loc[e];
                        }
                    }
                    lds_barrier();
#pragma unroll
                    for (int k = 0; k < CPW; ++k)
                        if (dg[k] < RD) sqb[hs[dg[k] * nch + wave + k * NW] + rk[k]] = ent[k];
                    lds_barrier();
                    int* tmp = sqa;
                    sqa = sqb;
                    sqb = tmp;
                }
                for (int i = tid; i < W; i += NT) ord_s[i] = sqa[i] & 1023;
            }
        }
        lds_barrier();
        if (!sharer && h == 0 && split == 0) {
            int* ord_hist = p.order_hist + ((size_t)slot * p.T_max + (t - 1)) * W;
            for (int i = tid; i < W; i += NT) {
                ord_next[i] = ord_s[i];
                ord_hist[i] = ord_s[i];
            }
        }
    }
    auto beam_at = [&](int i) __attribute__((always_inline)) { return track ? ord_s[i] : i; };
    auto posp = [&](int x) __attribute__((always_inline)) {
        return track ? (int)min((unsigned)posp_s[x], (unsigned)(W - 1)) : x;
    };

    // The replay is linear in the records, so instead of the sequential
    //   y <- alpha_j y + (k_j . x) delta_j      (j = oldest .. newest)
    // the kernel forms
    //   y = (prod_j alpha_j) S0 x + sum_j (k_j . x) (prod_{i>j} alpha_i) delta_j,
    // which makes the gathers of all depths independent: key gathers of
    // several depths are in flight together, and the newest block of delta
    // gathers is in flight during the projection MFMAs.
    // Streaming inputs of a chunk: k_t, q_t, v_t, alpha_t, beta_t, parents.
    // q, k, v are read once, so they carry the non-temporal hint: the caches
    // keep the records, which later chunks and later steps read again. (o is
    // written in 64-byte pieces by several waves and stays a normal store, so
    // the L2 merges the pieces into whole lines.)
    // (Two workgroups share a CU, 128 registers per lane each; latency is
    // hidden by the other workgroup rather than by prefetching in registers.)
    constexpr int SEG = DK / 8;                          // 16-byte pieces per k/q row
    constexpr int XITER = (2 * CH * SEG + NT - 1) / NT;
    constexpr int VSEG = DV / 8;                         // 16-byte pieces per v row
    constexpr int VITER = (CH * VSEG + NT - 1) / NT;
    u32x4 xv[XITER], vv[VITER];         // plain vector type: stays in registers
    float a_new = 0.f, b_new = 0.f;
    int par = 0;
    // Every gather and stream load below is issued unconditionally, from a
    // clamped address that is always inside its buffer (results for beams
    // past the end of the range are never used): with no branch around a
    // load, the compiler knows exactly how many loads are younger than the
    // one it waits for, and waits for no more than that.
    const int* parsrc = depth > 0 ? parin : reinterpret_cast<const int*>(ain);   // any valid int source at t = 1
    auto load_stream = [&](int cs, int tid) __attribute__((always_inline)) {
        const int last = min(CH, b_end - cs) - 1;
#pragma unroll
        for (int it = 0; it < XITER; ++it) {
            const int idx = tid + it * NT;
            const int row = idx / SEG, seg = idx % SEG;
            const bool is_k = row < CH;
            const int bl = min(is_k ? row : row - CH, last);
            xv[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>((is_k ? kin : qin) + beam_at(cs + bl) * HK + seg * 8));
        }
#pragma unroll
        for (int it = 0; it < VITER; ++it) {
            const int idx = tid + it * NT;
            const int bl = min(idx / VSEG, last), seg = idx % VSEG;
            vv[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vin + beam_at(cs + bl) * HV + seg * 8));
        }
        const int bq = min(tid, last);
        const int bb = beam_at(cs + bq);
        a_new = ain[bb * H];
        b_new = bin[bb * H];
        par = parsrc[bb];
    };

    for (int c0 = b_begin; c0 < b_end; c0 += CH) {
        const int nb = min(CH, b_end - c0);
        // Per-lane index values are re-derived every chunk from an opaque copy
        // of the thread id: cheaper than holding them (and the LDS addresses
        // made from them) in registers across the loop at 128 per lane.
        int tid_l = tid;
        asm volatile("" : "+v"(tid_l));
        const int n16 = tid_l & 15;                  // MFMA column within a 16-wide tile
        const int quad = (tid_l & 63) >> 4;          // which 4 rows of the wave's 16 this lane holds
        const int rbase = wave * kRowsPerWave + quad * 4;

        // ---- A. stage k_t, q_t, v_t, alpha_t, beta_t; ancestry rows ---------
        load_stream(c0, tid_l);
        const bool beam_thread = tid_l < nb;                   // one thread per beam of the chunk
        if (beam_thread && depth > 0) {
            if (par < 0 || par >= W) {                       // reported through the error word
                p.err[slot] = epoch;
                par = 0;
            }
            // the parent's row, kAncBatch entries per round: every load of a round is
            // issued (from clamped, in-row indices) before any is waited for, and stored
            // unconditionally (entries past the row land in row depth-1, written last)
            const int* src = anc_prev + par * p.T_max;
            for (int j0 = 0; j0 + 1 < depth; j0 += kAncBatch) {
                int row[kAncBatch];
#pragma unroll
                for (int u = 0; u < kAncBatch; ++u) row[u] = src[min(j0 + u, depth - 2)];
#pragma unroll
                for (int u = 0; u < kAncBatch; ++u) anc_s[min(j0 + u, depth - 1) * CH + tid_l] = row[u];
            }
            anc_s[(depth - 1) * CH + tid_l] = (depth - 1) * W + posp(par);   // parent's own record of step t-1
        }
        if constexpr (FUSED) {
            // a row's SEG pieces sit in SEG adjacent lanes of one wave
            static_assert((2 * CH * SEG) % NT == 0 && 64 % SEG == 0, "whole rows per wave");
#pragma unroll
            for (int it = 0; it < XITER; ++it) {
                float x[8], ss = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = bf_lo(xv[it][e]);
                    x[2 * e + 1] = bf_hi(xv[it][e]);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
                for (int m = 1; m < SEG; m <<= 1) ss += __shfl_xor(ss, m, 64);
                const float inv = 1.f / sqrtf(ss + p.norm_eps);
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[it][e] = pack_bf16x2(x[2 * e] * inv, x[2 * e + 1] * inv);
            }
        }
#pragma unroll
        for (int it = 0; it < XITER; ++it) {
            const int idx = tid_l + it * NT;
            if (idx < 2 * CH * SEG) {
                const int row = idx / SEG, seg = idx % SEG;
                *reinterpret_cast<u32x4*>(xs + row * XS + seg * 8) = xv[it];
            }
        }
#pragma unroll
        for (int it = 0; it < VITER; ++it) {
            const int idx = tid_l + it * NT;
            if (idx < CH * VSEG) {
                const int bl = idx / VSEG, seg = idx % VSEG;
                *reinterpret_cast<u32x4*>(vs + bl * VS + seg * 8) = vv[it];
            }
        }
        if (beam_thread) {
            const float at = FUSED ? gate_alpha(a_new, neg_A, dtb) : a_new;
            at_s[tid_l] = at;
            bt_s[tid_l] = FUSED ? gate_beta(b_new) : b_new;
            ralpha[depth * W + c0 + tid_l] = at;          // alpha_t record, at the beam's position
        }
        lds_barrier();

        // ---- B. k_j . k_t and k_j . q_t for every ancestral record j -------
        // On the matrix cores: for a tile of 16 beams and one depth, the A
        // operand is the 16 ancestral keys, gathered from the record store
        // straight into A-fragments, and B holds the same beams' k_t (or q_t)
        // columns from LDS; the wanted dot products are the diagonal of the
        // 16x16 product, whose element (i, i) sits in lane i + 16*(i/4),
        // register i%4.
        const int n_units = MT * depth;
        const bool diag = (n16 >> 2) == quad;
        bf16x8 af[UPP][KS];
        int rid[UPP];
        float aj[UPP];
        auto issue_units = [&](int u0) __attribute__((always_inline)) {   // units u0, u0 + NW, ... of this wave
#pragma unroll
            for (int h2 = 0; h2 < UPP; ++h2) {
                const int u = u0 + h2 * NW;
                const int m = u % MT, j = u / MT;
                const int bl = m * 16 + n16;
                rid[h2] = (u < n_units && bl < nb) ? anc_s[j * CH + bl] : 0;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    af[h2][kk] = *reinterpret_cast<const bf16x8*>(rkey + rid[h2] * DK + kk * 32 + quad * 8);
                aj[h2] = ralpha[rid[h2]];
            }
        };
        auto consume_units = [&](int u0) __attribute__((always_inline)) {
#pragma unroll
            for (int h2 = 0; h2 < UPP; ++h2) {
                const int u = u0 + h2 * NW;
                if (u >= n_units) break;                     // uniform across the wave
                const int m = u % MT, j = u / MT;
                f32x4 dk4 = f32x4{0.f, 0.f, 0.f, 0.f}, dq4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const int koff = kk * 32 + quad * 8;
                    const bf16x8 bk = *reinterpret_cast<const bf16x8*>(xs + (m * 16 + n16) * XS + koff);
                    const bf16x8 bq = *reinterpret_cast<const bf16x8*>(xs + (CH + m * 16 + n16) * XS + koff);
                    dk4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[h2][kk], bk, dk4, 0, 0, 0);
                    dq4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[h2][kk], bq, dq4, 0, 0, 0);
                }
                const int bl = m * 16 + n16;
                if (diag && bl < nb) {
                    const int r = n16 & 3;
                    const float dk = r == 0 ? dk4[0] : r == 1 ? dk4[1] : r == 2 ? dk4[2] : dk4[3];
                    const float dq = r == 0 ? dq4[0] : r == 1 ? dq4[1] : r == 2 ? dq4[2] : dq4[3];
                    coef_s[j * CH + bl] = make_float4(dk, dq, aj[h2], __int_as_float(rid[h2]));
                }
            }
        };
        if constexpr (HIST) {
            issue_units(wave);
            consume_units(wave);
            for (int u0 = wave + UPP * NW; u0 < n_units; u0 += UPP * NW) {   // deeper histories
                issue_units(u0);
                consume_units(u0);
            }
        }
        {   // k_t . q_t on the vector units, from LDS
            const int bl = min(tid_l / TPQ, CH - 1), part = tid_l % TPQ;   // (threads past the chunk repeat its last beam)
            const uint16_t* kt_s = xs + bl * XS + part * EQ;
            const uint16_t* qt_s = xs + (CH + bl) * XS + part * EQ;
            float kq = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < EQ / 8; ++s2)
                kq = dot8(*reinterpret_cast<const uint4*>(kt_s + s2 * 8), *reinterpret_cast<const uint4*>(qt_s + s2 * 8), kq);
#pragma unroll
            for (int m = 1; m < TPQ; m <<= 1) kq += __shfl_xor(kq, m, 64);
            if (part == 0 && tid_l / TPQ < nb) kq_s[bl] = kq;
        }

        lds_barrier();   // coef_s / kq_s complete

        // ---- C + D, one 32-beam group at a time ------------------------------
        // Lane l handles beams g*32 + l%16 and g*32 + 16 + l%16 of the chunk
        // and rows rbase .. rbase+3: the 16x16 MFMA accumulator register i of
        // lane l holds row 4*(l/16) + i (of the wave's 16) for column l%16.
#pragma unroll 1
        for (int g = 0; g < NG; ++g) {
            // the newest DBD ancestral deltas of the lane's two beams, in flight
            // during the projection MFMAs
            float4 dd[2][DBD];
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                const int bl = g * 32 + u2 * 16 + n16;
#pragma unroll
                for (int u = 0; u < DBD; ++u) {
                    const int j = depth - 1 - u;
                    const int r = (bl < nb && j >= 0) ? anc_s[j * CH + bl] : 0;
                    if constexpr (HIST) dd[u2][u] = *reinterpret_cast<const float4*>(rdw + r * DV + quad * 4);
                    else dd[u2][u] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
            f32x4 acc[4];                  // tiles: k of beams +0..15, k +16..31, q +0..15, q +16..31
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int col = (ct >= 2 ? CH : 0) + g * 32 + (ct & 1) * 16 + n16;
                    const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(xs + col * XS + kk * 32 + quad * 8);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi[kk], bfr, acc[ct], 0, 0, 0);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo[kk], bfr, acc[ct], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);   // keep B-fragment reads next to their k-step
            }
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                const int bl = g * 32 + u2 * 16 + n16;
                if (bl >= nb) continue;
                // newest record first: w_j = (k_j . x) * prod_{i>j} alpha_i
                f32x4 zk = f32x4{0.f, 0.f, 0.f, 0.f}, zq = f32x4{0.f, 0.f, 0.f, 0.f};
                float sfx = 1.f;
                for (int jt = depth - 1; jt >= 0; jt -= DBD) {
                    if (jt != depth - 1) {                           // older blocks (depth > DBD)
#pragma unroll
                        for (int u = 0; u < DBD; ++u)
                            if (jt - u >= 0)
                                dd[u2][u] = *reinterpret_cast<const float4*>(
                                    rdw + anc_s[(jt - u) * CH + bl] * DV + quad * 4);
                    }
#pragma unroll
                    for (int u = 0; u < DBD; ++u) {
                        if (jt - u >= 0) {
                            const float4 c = coef_s[(jt - u) * CH + bl];
                            const float4 dv4 = dd[u2][u];
                            const float wk = c.x * sfx, wq = c.y * sfx;
                            sfx *= c.z;
                            zk[0] = fmaf(wk, dv4.x, zk[0]);
                            zk[1] = fmaf(wk, dv4.y, zk[1]);
                            zk[2] = fmaf(wk, dv4.z, zk[2]);
                            zk[3] = fmaf(wk, dv4.w, zk[3]);
                            zq[0] = fmaf(wq, dv4.x, zq[0]);
                            zq[1] = fmaf(wq, dv4.y, zq[1]);
                            zq[2] = fmaf(wq, dv4.z, zq[2]);
                            zq[3] = fmaf(wq, dv4.w, zq[3]);
                        }
                    }
                }
                // sfx is now the product of alpha over the whole history
                const f32x4 yk = acc[u2] * sfx + zk, yq = acc[2 + u2] * sfx + zq;
                const int b = beam_at(c0 + bl);
                const float kq = kq_s[bl], a = at_s[bl], bb = bt_s[bl];
                const uint2 vb = *reinterpret_cast<const uint2*>(vs + bl * VS + rbase);
                float4 d, o;
                d.x = bb * (bf_lo(vb.x) - a * yk[0]);
                d.y = bb * (bf_hi(vb.x) - a * yk[1]);
                d.z = bb * (bf_lo(vb.y) - a * yk[2]);
                d.w = bb * (bf_hi(vb.y) - a * yk[3]);
                o.x = fmaf(a, yq[0], kq * d.x);
                o.y = fmaf(a, yq[1], kq * d.y);
                o.z = fmaf(a, yq[2], kq * d.z);
                o.w = fmaf(a, yq[3], kq * d.w);
                if constexpr (FUSED)
                    *reinterpret_cast<uint2*>(oout16 + b * HV + rbase) =
                        make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
                else
                    *reinterpret_cast<float4*>(oout + b * HV + rbase) = o;
                *reinterpret_cast<float4*>(rdw + (depth * W + c0 + bl) * DV + quad * 4) = d;
                if (dout) *reinterpret_cast<float4*>(dout + b * HV + rbase) = d;
            }
        }

        // ---- append k_t (whole 256-byte rows) after every gather ------------
#pragma unroll
        for (int it = 0; it < XITER; ++it) {
            const int idx = tid_l + it * NT;
            const int row = idx / SEG, seg = idx % SEG;
            if (idx < 2 * CH * SEG && row < nb)
                *reinterpret_cast<uint4*>(rkey + (depth * W + c0 + row) * DK + seg * 8) =
                    *reinterpret_cast<const uint4*>(xs + row * XS + seg * 8);
        }
        lds_barrier();   // LDS is reused by the next chunk
    }

    // ---- the request's new index rows, in beam-index order over this
    // workgroup's index range (the splits of a (request, head) cover [0, W)
    // between them), so the small writes coalesce.
    if (p.write_index && h == 0 && depth > 0) {   // one head of the index owner writes it
        for (int b = b_begin + tid; b < b_end; b += NT) {
            int pb = parin[b];
            pb = (pb < 0 || pb >= W) ? 0 : pb;         // (reported in phase A)
            for (int j0 = 0; j0 + 1 < depth; j0 += kAncBatch) {   // (as the phase-A copy)
                int row[kAncBatch];
#pragma unroll
                for (int u = 0; u < kAncBatch; ++u) row[u] = anc_prev[pb * p.T_max + min(j0 + u, depth - 2)];
#pragma unroll
                for (int u = 0; u < kAncBatch; ++u) anc_next[b * p.T_max + min(j0 + u, depth - 1)] = row[u];
            }
            anc_next[b * p.T_max + depth - 1] = (depth - 1) * W + posp(pb);
        }
    }
    count_done();
}

// The workgroup's (request, head, beam range), as step_body derives it.
__device__ __forceinline__ int step_request(const StepParams& p) {
    int L = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) L = (L & 7) * (nblk >> 3) + (L >> 3);
    return L / p.n_splits / p.H;
}

// MODE kStepFirst: every request of the launch is at its first step;
// kStepHist: none is; kStepAny: each workgroup takes the body without record
// gathers when its request is at its first step, which the host cannot know
// in graph mode (the step index lives on the device). The two bodies in one
// kernel raise its register pressure, so uniform launches keep their own.
template <int DK, int DV, bool FUSED, int MODE, int HCH>
__global__ __launch_bounds__(step_threads<DV>()) __attribute__((amdgpu_waves_per_eu(4))) void step_kernel(const StepParams p) {
    if constexpr (MODE == kStepAny) {
        const int ri = step_request(p);
        const int t = p.dev_steps ? p.dev_steps[p.slot[ri]] + 1 : p.t[ri];
        if (t <= 1) step_body<DK, DV, FUSED, false, HCH>(p);
        else step_body<DK, DV, FUSED, true, HCH>(p);
    } else {
        step_body<DK, DV, FUSED, MODE == kStepHist, HCH>(p);
    }
}

template <int DK, int DV>
hipError_t launch_init_t(const float* S0, uint16_t* planes, int H, hipStream_t s) {
    const int n = H * DV * DK / 8;
    hipLaunchKernelGGL((init_s0_kernel<DK, DV>), dim3((n + 255) / 256), dim3(256), 0, s, S0, planes, H);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t prepare_step_t(int T_max, int W) {
    const size_t lds = step_lds_bytes(DK, DV, T_max, W);
    if (lds <= 65536) return hipSuccess;
    constexpr int S = kChunk / 2;
    const void* kernels[] = {
        reinterpret_cast<const void*>(&step_kernel<DK, DV, false, kStepFirst, kChunk>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, false, kStepHist, kChunk>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, false, kStepAny, kChunk>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, false, kStepHist, S>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, false, kStepAny, S>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, true, kStepFirst, kChunk>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, true, kStepHist, kChunk>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, true, kStepAny, kChunk>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, true, kStepHist, S>),
        reinterpret_cast<const void*>(&step_kernel<DK, DV, true, kStepAny, S>)};
    for (const void* k : kernels) {
        const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, int DV, bool FUSED, int HCH>
void launch_step_mode(int mode, dim3 grid, dim3 block, size_t lds, const StepParams& p, hipStream_t s) {
    if (mode == kStepFirst) hipLaunchKernelGGL((step_kernel<DK, DV, FUSED, kStepFirst, kChunk>), grid, block, lds, s, p);
    else if (mode == kStepHist) hipLaunchKernelGGL((step_kernel<DK, DV, FUSED, kStepHist, HCH>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((step_kernel<DK, DV, FUSED, kStepAny, HCH>), grid, block, lds, s, p);
}

template <int DK, int DV>
hipError_t launch_step_t(bool fused, int mode, bool half_chunks, const StepParams& p, hipStream_t s) {
    const size_t lds = step_lds_bytes(DK, DV, p.T_max, p.W);
    const dim3 grid(p.n_req * p.H * p.n_splits), block(step_threads<DV>());
    if (half_chunks) {
        if (fused) launch_step_mode<DK, DV, true, kChunk / 2>(mode, grid, block, lds, p, s);
        else launch_step_mode<DK, DV, false, kChunk / 2>(mode, grid, block, lds, p, s);
    } else {
        if (fused) launch_step_mode<DK, DV, true, kChunk>(mode, grid, block, lds, p, s);
        else launch_step_mode<DK, DV, false, kChunk>(mode, grid, block, lds, p, s);
    }
    return hipGetLastError();
}

__global__ __launch_bounds__(64) void set_counters_kernel(int32_t* steps, int32_t* epoch, int req, int sv, int ev) {
    if (threadIdx.x == 0) {
        steps[req] = sv;
        epoch[req] = ev;
    }
}

}  // namespace

size_t step_lds_bytes(int dk, int dv, int T_max, int W) {
    const size_t ms = T_max > 1 ? (size_t)T_max - 1 : 1;
    return kChunk * ms * 16                       // coef_s
           + 2 * kChunk * (size_t)(dk + 16) * 2   // xs
           + kChunk * (size_t)(dv + 16) * 2       // vs
           + kChunk * ms * 4                      // anc_s
           + 3 * kChunk * 4                       // kq_s, at_s, bt_s
           + (W <= kOrderMax ? 2 * (size_t)((W + 3) & ~3) * 4 : 0);   // ord_s, posp_s
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

hipError_t prepare_step(int dk, int dv, int T_max, int W) {
    if (dk == 32 && dv == 32) return prepare_step_t<32, 32>(T_max, W);
    if (dk == 64 && dv == 64) return prepare_step_t<64, 64>(T_max, W);
    if (dk == 128 && dv == 128) return prepare_step_t<128, 128>(T_max, W);
    return hipErrorInvalidValue;
}

hipError_t launch_set_counters(int32_t* dev_steps, int32_t* dev_epoch, int req, int steps_value, int epoch_value,
                               hipStream_t s) {
    hipLaunchKernelGGL(set_counters_kernel, dim3(1), dim3(64), 0, s, dev_steps, dev_epoch, req, steps_value,
                       epoch_value);
    return hipGetLastError();
}

hipError_t launch_step(int dk, int dv, bool fused, int mode, bool half_chunks, const StepParams& p, hipStream_t s) {
    if (mode != kStepFirst && mode != kStepHist && mode != kStepAny) return hipErrorInvalidValue;
    if (half_chunks && p.beams_per_block % (kChunk / 2) != 0) return hipErrorInvalidValue;
    if (!half_chunks && p.beams_per_block % kChunk != 0 && p.beams_per_block < p.W) return hipErrorInvalidValue;
    if (dk == 32 && dv == 32) return launch_step_t<32, 32>(fused, mode, half_chunks, p, s);
    if (dk == 64 && dv == 64) return launch_step_t<64, 64>(fused, mode, half_chunks, p, s);
    if (dk == 128 && dv == 128) return launch_step_t<128, 128>(fused, mode, half_chunks, p, s);
    return hipErrorInvalidValue;
}

}  // namespace onela
