// select.hip - Quest block metadata, selection (scoring + top-K with M = A \ P) and predictor kernels
// (gfx950).  The scoring, top-K and predictor device code, its design notes and citations are in
// select_core.hpp; the metadata kernel is here.
//
// Citations:
//   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
//           Decoding" (full paper text)

#include <type_traits>

#include "select_core.hpp"
#include "kv_types.hpp"

namespace prr {
namespace {

// ------------------------------------------------------------------------------------------------
// Block metadata
// ------------------------------------------------------------------------------------------------

struct MetaParams {
    const void *k;
    const int32_t *page_table;
    const int32_t *seq_len;
    void *meta;
    int hkv, max_pages, num_pages, block, stride, nmax;
};

// 16 bytes of K at element offset off: the channels they hold as floats (4 for f32, 8 for bf16, 16
// for fp8), exactly.  The load and the widening are separate steps so that a kernel can issue a run of
// loads before it widens any of them.
template <int KT>
constexpr int kElemsPer16B = KT == kKtF32 ? 4 : KT == kKtBf16 ? 8 : 16;

// The loads are non-temporal: the summary kernels read every K row once.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int KT>
__device__ __forceinline__ uint4 load16_raw(const void *k, size_t off) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)((const uint8_t *)k + off * (16 / kElemsPer16B<KT>)));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int KT>
__device__ __forceinline__ void widen16(const uint4 raw, float (&x)[kElemsPer16B<KT>]) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (KT == kKtF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
    } else if constexpr (KT == kKtBf16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float f[4];
            fp8x4_to_f32(w[q], f);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * q + e] = f[e];
        }
    }
}

// Block summaries of the K cache, written once at prefill.
//  - Quest min/max metadata (MEAN = false): [B][Hkv][d][2][stride], the channel-wise minimum and maximum
//    key of every block; fp32 for an f32 cache, bf16 otherwise (an fp8 key is a bf16 value, so its min
//    and max are too).
//  - Mean-pooled summary (MEAN = true): [B][Hkv][d][stride] fp32, the channel-wise mean key of every
//    block over its valid tokens, summed in float64 in token order, divided by the token count and
//    rounded once to float32.
// A workgroup covers 64 consecutive blocks of one (sequence, kv head).  A group of G = d / EPL lanes reads
// one token row of one block per 16-byte-per-lane load (each lane holds EPL channels), so a wave walks
// 64 / G blocks at once, each lane through its block's tokens in order, with a whole page's loads in
// flight and the next page's id fetched ahead of them.  The summaries go to LDS and the workgroup writes
// each output row of its 64 blocks as one contiguous run.
template <int KT>
using MetaElem = typename std::conditional<KT == kKtF32, float, uint16_t>::type;

template <int KT>
__device__ __forceinline__ MetaElem<KT> meta_value(float x) {
    if constexpr (KT == kKtF32) return x;
    else return (uint16_t)(__float_as_uint(x) >> 16);   // a bf16 value: its top 16 bits, exactly
}

template <int KT, int D, bool MEAN>
__global__ __launch_bounds__(256) void summary_kernel(MetaParams p) {
    constexpr int EPL = kElemsPer16B<KT>;   // channels per 16-byte load
    constexpr int G = D / EPL;              // lanes per token row
    constexpr int BPW = 64 / G;             // blocks a wave walks at once
    static_assert(64 % (4 * BPW) == 0, "the waves' block rounds tile the workgroup's 64 blocks");
    using OT = typename std::conditional<MEAN, float, MetaElem<KT>>::type;
    constexpr int ROWS = MEAN ? 1 : 2;      // output rows per channel
    // [row][block][channel], padded to an odd number of 32-bit words per block so that an output row's
    // reads by consecutive blocks fall on distinct LDS banks
    constexpr int PAD = sizeof(OT) == 4 ? 1 : 2;
    __shared__ OT s_out[ROWS][64][D + PAD];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int u = blockIdx.y;
    const int b = u / p.hkv, kvh = u - b * p.hkv;
    const int slen = min(max(p.seq_len[b], 0), p.max_pages * kPage);
    const int nb = min((slen + p.block - 1) / p.block, p.nmax);
    const int blk0 = blockIdx.x * 64;
    if (blk0 >= nb) return;                 // the whole workgroup
    const int *prow = p.page_table + (size_t)b * p.max_pages;
    const int g = lane % G, sub = lane / G;
    // the id of the page the lane's group reads next, fetched a page ahead (also across rounds)
    int ph_next = prow[min((blk0 + wave * BPW + sub) * p.block, slen - 1) / kPage];
    for (int r = wave * BPW; r < 64; r += 4 * BPW) {
        const int bi = r + sub;
        if (blk0 + bi >= nb) continue;
        const int t0 = (blk0 + bi) * p.block;
        const int t1 = min(t0 + p.block, slen);
        float mn[EPL], mx[EPL];
        double acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            mn[e] = INFINITY;
            mx[e] = -INFINITY;
            acc[e] = 0.0;
        }
        for (int tp = t0; tp < t1; tp += kPage) {   // a block starts on a page boundary
            const int ph = min(max(ph_next, 0), p.num_pages - 1);
            // next: this block's next page, else the first page of the group's block in the next round
            const int tn = tp + kPage < t1 ? tp + kPage : t0 + 4 * BPW * p.block;
            ph_next = prow[min(tn, slen - 1) / kPage];
            const size_t pbase = ((size_t)ph * p.hkv + kvh) * kPage * D + (size_t)g * EPL;
            const int n = min(kPage, t1 - tp);
            uint4 raw[kPage];
            // all of the page's loads first; a ragged page repeats its last row, which a minimum or
            // maximum absorbs and the sum skips
#pragma unroll
            for (int i = 0; i < kPage; ++i) raw[i] = load16_raw<KT>(p.k, pbase + (size_t)min(i, n - 1) * D);
#pragma unroll
            for (int i = 0; i < kPage; ++i) {
                float x[EPL];
                widen16<KT>(raw[i], x);
                if constexpr (MEAN) {
                    if (i < n) {
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[e] = dadd(acc[e], (double)x[e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        mn[e] = fminf(mn[e], x[e]);
                        mx[e] = fmaxf(mx[e], x[e]);
                    }
                }
            }
        }
        if constexpr (MEAN) {
            const double cnt = (double)(t1 - t0);
#pragma unroll
            for (int e = 0; e < EPL; ++e) s_out[0][bi][g * EPL + e] = (float)(acc[e] / cnt);
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                s_out[0][bi][g * EPL + e] = meta_value<KT>(mn[e]);
                s_out[ROWS - 1][bi][g * EPL + e] = meta_value<KT>(mx[e]);
            }
        }
    }
    __syncthreads();
    // output row q = channel * ROWS + (0: min or mean, 1: max), 64 consecutive blocks per row
    const int nblk = min(64, nb - blk0);
    OT *out = (OT *)p.meta;
    for (int it = threadIdx.x; it < ROWS * D * 64; it += 256) {
        const int q = it / 64, bi = it % 64;
        if (bi < nblk) out[((size_t)u * D * ROWS + q) * p.stride + blk0 + bi] = s_out[q % ROWS][bi][q / ROWS];
    }
}

// ------------------------------------------------------------------------------------------------
// Kernels
// ------------------------------------------------------------------------------------------------

template <bool BF16, int D, bool MEAN, int BPL = kScoreBPL<BF16, MEAN>>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
    double kept[BPL];
    score_body<BF16, D, false, MEAN, BPL>(p, blockIdx.x, blockIdx.y, kept);
}

// First stage of a three-stage top-K over rows longer than one top-K workgroup holds: workgroup bx of
// unit u scores its 256 BPL blocks and keeps their local top-kl as candidates (stages two and three in
// topk_groups_kernel).  BPL: kScoreBPL, or kWideScoreBPL for the bf16 min/max parts of long rows.
template <bool BF16, int D, bool MEAN, int BPL = kScoreBPL<BF16, MEAN>>
__global__ __launch_bounds__(256) void score_parts_kernel(ScoreParams p, CandParams cp, int nsx) {
    __shared__ TopkSmem<4> sm;
    constexpr int BPW = 256 * BPL;
    const int bx = blockIdx.x, u = blockIdx.y;
    double kept[BPL] = {};
    score_body<BF16, D, false, MEAN, BPL>(p, bx, u, kept);
    const int b = u / p.hkv;
    const int nb = min((max(p.seq_len[b], 0) + p.block - 1) / p.block, p.nmax);
    const int n_local = min(max(nb - bx * BPW, 0), BPW);
    const size_t part = (size_t)u * nsx + bx;
    local_candidates<BPL>(kept, n_local, cp.kl, bx * BPW, cp.key + part * cp.kl, cp.idx + part * cp.kl,
                          cp.cnt + part, sm);
}

template <int KPT, int TPB>
__global__ __launch_bounds__(TPB) void topk_kernel(TopkParams p) {
    topk_body<KPT, TPB>(p, blockIdx.x);
}

template <int KPT, int TPB>
__global__ __launch_bounds__(TPB) void predict_kernel(PredictParams p) {
    predict_body<KPT, TPB>(p, blockIdx.x);
}

// Long predictor rows: grid (parts, units) of 256 threads; the last part of a unit to arrive (a
// device-scope counter, reset by it) ranks the unit's candidates, KPT slots per thread.
template <int KPT>
__global__ __launch_bounds__(256) void predict_parts_kernel(PredictParams p, TopkParams tp, CandParams cp,
                                                            uint32_t *arrivals, int nparts) {
    __shared__ TopkSmem<4> sm;
    __shared__ int s_last;
    const int part = blockIdx.x, u = blockIdx.y;
    const size_t pi = (size_t)u * nparts + part;
    predict_part_body(p, u, part, cp.key + pi * cp.kl, cp.idx + pi * cp.kl, cp.cnt + pi, cp.kl, sm);
    // this workgroup's state and candidate stores are complete before its arrival is counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&arrivals[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(nparts - 1);
        if (s_last) __hip_atomic_store(&arrivals[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (s_last) {
        topk_candidates_body<KPT>(tp, u, cp.key + (size_t)u * nparts * cp.kl, cp.idx + (size_t)u * nparts * cp.kl,
                                  cp.cnt + (size_t)u * nparts, nparts, cp.kl);
        if (threadIdx.x == 0) {
            const int b = u / p.hkv;
            p.live[u] = min((p.seq_len[b] + p.block - 1) / p.block, p.nmax);
        }
    }
}

// Second and third stages of a three-stage top-K: grid (groups, units) of 256 threads.  Group g of unit
// u keeps the top-kl2 of the candidates of parts [g gp, (g + 1) gp); the unit's last group to arrive (a
// device-scope counter, reset by it) ranks the groups' candidates into A and M.
template <int KPT2, int KPT3>
__global__ __launch_bounds__(256) void topk_groups_kernel(TopkParams tp, CandParams c1, CandParams c2,
                                                          uint32_t *arrivals, int nparts, int gp, int ng,
                                                          int32_t *live) {
    __shared__ int s_last;
    const int g = blockIdx.x, u = blockIdx.y;
    const int p0 = g * gp;
    const int gparts = min(gp, nparts - p0);
    const size_t in = (size_t)u * nparts + p0;
    const size_t out = (size_t)u * ng + g;
    group_candidates<KPT2>(c1.key + in * c1.kl, c1.idx + in * c1.kl, c1.cnt + in, gparts, c1.kl, c2.kl,
                           c2.key + out * c2.kl, c2.idx + out * c2.kl, c2.cnt + out);
    // this group's candidate stores are complete before its arrival is counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&arrivals[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(ng - 1);
        if (s_last) __hip_atomic_store(&arrivals[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (s_last) {
        topk_candidates_body<KPT3, false, kMaxSelectN>(tp, u, c2.key + (size_t)u * ng * c2.kl, c2.idx + (size_t)u * ng * c2.kl,
                                   c2.cnt + (size_t)u * ng, ng, c2.kl);
        if (live && threadIdx.x == 0) {   // a predictor step: its blocks are all live from now on
            const int b = u / tp.hkv;
            live[u] = min((tp.seq_len[b] + tp.block - 1) / tp.block, tp.nmax);
        }
    }
}

// First stage of a three-stage predictor step: part `part` of unit u updates its blocks' EMA state and
// keeps its local candidates (predict_part_body); the groups follow in topk_groups_kernel.
__global__ __launch_bounds__(256) void predict_parts_only_kernel(PredictParams p, CandParams cp, int nparts) {
    __shared__ TopkSmem<4> sm;
    const int part = blockIdx.x, u = blockIdx.y;
    const size_t pi = (size_t)u * nparts + part;
    predict_part_body(p, u, part, cp.key + pi * cp.kl, cp.idx + pi * cp.kl, cp.cnt + pi, cp.kl, sm);
}

template <template <int, int> class Launch, typename P>
hipError_t dispatch_topk(int nmax, int units, const P &p, hipStream_t stream) {
    int tpb, kpt;
    topk_shape(nmax, tpb, kpt);
#define PRR_CASE(T, K) \
    if (tpb == T && kpt == K) return Launch<K, T>::run(units, p, stream);
    PRR_CASE(64, 1) PRR_CASE(64, 2) PRR_CASE(256, 1) PRR_CASE(256, 2) PRR_CASE(256, 4)
    PRR_CASE(1024, 2) PRR_CASE(1024, 4) PRR_CASE(1024, 8) PRR_CASE(1024, 16) PRR_CASE(1024, 32)
#undef PRR_CASE
    return hipErrorInvalidValue;
}

template <int KPT, int TPB>
struct TopkLaunch {
    static hipError_t run(int units, const TopkParams &p, hipStream_t stream) {
        PRR_LAUNCH(topk_kernel<KPT, TPB>, dim3(units), dim3(TPB), stream, p);
        return hipGetLastError();
    }
};

template <int KPT, int TPB>
struct PredictLaunch {
    static hipError_t run(int units, const PredictParams &p, hipStream_t stream) {
        PRR_LAUNCH(predict_kernel<KPT, TPB>, dim3(units), dim3(TPB), stream, p);
        return hipGetLastError();
    }
};

}  // namespace

hipError_t launch_meta(const KvDesc &kv, int block, int stride, void *meta, bool mean, hipStream_t stream) {
    MetaParams p{};
    p.k = kv.k;
    p.page_table = kv.page_table;
    p.seq_len = kv.seq_len;
    p.meta = meta;
    p.hkv = kv.hkv;
    p.max_pages = kv.max_pages;
    p.num_pages = kv.num_pages;
    p.block = block;
    p.stride = stride;
    p.nmax = (int)((long)kv.max_pages * kPage / block);
    const dim3 grid((p.nmax + 63) / 64, kv.batch * kv.hkv);
    const int kt = kv.fp8 ? kKtFp8 : kv.bf16 ? kKtBf16 : kKtF32;
#define PRR_META(KT, DD)                                                                             \
    if (kt == KT && kv.d == DD) {                                                                    \
        if (mean) PRR_LAUNCH((summary_kernel<KT, DD, true>), dim3(grid), dim3(256), stream, p);     \
        else PRR_LAUNCH((summary_kernel<KT, DD, false>), dim3(grid), dim3(256), stream, p);         \
    } else
    PRR_META(kKtF32, 128) PRR_META(kKtF32, 64) PRR_META(kKtBf16, 128) PRR_META(kKtBf16, 64)
    PRR_META(kKtFp8, 128) PRR_META(kKtFp8, 64)
    { return hipErrorInvalidValue; }
#undef PRR_META
    return hipGetLastError();
}

hipError_t launch_select(const KvDesc &kv, const void *q, int hq, const void *meta, int block,
                         int stride, int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt,
                         int p_cap, double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap,
                         int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap, bool mean, void *ws,
                         hipStream_t stream) {
    const int units = kv.batch * kv.hkv;
    ScoreParams sp;
    sp.q = q;
    sp.meta = meta;
    sp.seq_len = kv.seq_len;
    sp.scores = scores;
    sp.hq = hq;
    sp.hkv = kv.hkv;
    sp.G = hq / kv.hkv;
    sp.block = block;
    sp.stride = stride;
    sp.nmax = nmax;
    const bool bq = kv.bf16 || kv.fp8;   // bf16 queries (and bf16 min/max metadata)
    const SelectSpecPlan plan = ws && nmax > kStagedSelectMin ? select_stage_plan(nmax, topk, bq, mean) : SelectSpecPlan{};
    if (nmax > kMaxRowTopK && !plan.three) return hipErrorInvalidValue;
    // The score kernel alone scores one bf16 min/max block per lane: twice the workgroups of the fused
    // launches' two per lane (whose grid shares the chip with the speculative pass), two waves per SIMD
    // to hide each other's float64 chains.  128K, batch 8: selection 21.7 -> 18.9 us; 32K: 18.7 -> 14.8 us.
    const bool one_per_lane = bq && !mean;
    const int bpw = plan.three ? plan.bpw : one_per_lane ? 256 : score_bpw(bq, mean);
    const dim3 sgrid((nmax + bpw - 1) / bpw, units);
    if (plan.three) {
        // three stages: the scoring workgroups keep their parts' candidates, then groups and the ranking
        const int nsx = (int)sgrid.x;
        const StageLayout sl = stage_layout((char *)ws, units, nsx, plan);
        CandParams cp;
        cp.key = (uint64_t *)sl.cand1;
        cp.idx = (int32_t *)(sl.cand1 + (size_t)units * nsx * plan.kl * 8);
        cp.cnt = (int32_t *)(sl.cand1 + (size_t)units * nsx * plan.kl * 12);
        cp.kl = plan.kl;
        const bool wide = plan.bpw == score_bpw(true, false, true);
        if (wide && kv.d == 128) PRR_LAUNCH((score_parts_kernel<true, 128, false, kWideScoreBPL>), dim3(sgrid), dim3(256), stream, sp, cp, nsx);
        else if (wide && kv.d == 64) PRR_LAUNCH((score_parts_kernel<true, 64, false, kWideScoreBPL>), dim3(sgrid), dim3(256), stream, sp, cp, nsx);
        else
#define PRR_SP(BQ, DD, MN)                                                                                   \
        if (bq == BQ && kv.d == DD && mean == MN) PRR_LAUNCH((score_parts_kernel<BQ, DD, MN>), dim3(sgrid), dim3(256), stream, sp, cp, nsx); \
        else
        PRR_SP(true, 128, false) PRR_SP(true, 64, false) PRR_SP(false, 128, false) PRR_SP(false, 64, false)
        PRR_SP(true, 128, true) PRR_SP(true, 64, true) PRR_SP(false, 128, true) PRR_SP(false, 64, true)
        { return hipErrorInvalidValue; }
#undef PRR_SP
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_topk_groups(kv, block, nmax, topk, p_idx, p_cnt, p_cap, a_idx, a_cnt, nullptr, a_cap, m_idx, m_cnt,
                                  m_pages, m_cap, plan, nsx, sl.cand1, sl.cand2, sl.garr, stream);
    }
    if (mean) {
        // the fp32 block means do not depend on the cache dtype beyond q's
        if (bq) {
            if (kv.d == 128) PRR_LAUNCH(score_kernel<true, 128, true>, dim3(sgrid), dim3(256), stream, sp);
            else PRR_LAUNCH(score_kernel<true, 64, true>, dim3(sgrid), dim3(256), stream, sp);
        } else {
            if (kv.d == 128) PRR_LAUNCH(score_kernel<false, 128, true>, dim3(sgrid), dim3(256), stream, sp);
            else PRR_LAUNCH(score_kernel<false, 64, true>, dim3(sgrid), dim3(256), stream, sp);
        }
    } else if (bq) {
        if (kv.d == 128) PRR_LAUNCH((score_kernel<true, 128, false, 1>), dim3(sgrid), dim3(256), stream, sp);
        else PRR_LAUNCH((score_kernel<true, 64, false, 1>), dim3(sgrid), dim3(256), stream, sp);
    } else {
        if (kv.d == 128) PRR_LAUNCH(score_kernel<false, 128, false>, dim3(sgrid), dim3(256), stream, sp);
        else PRR_LAUNCH(score_kernel<false, 64, false>, dim3(sgrid), dim3(256), stream, sp);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk(kv, block, nmax, topk, scores, p_idx, p_cnt, p_cap, a_idx, a_cnt, a_cap, m_idx, m_cnt,
                       m_pages, m_cap, stream);
}

hipError_t launch_topk(const KvDesc &kv, int block, int nmax, int topk, const double *scores,
                       const int32_t *p_idx, const int32_t *p_cnt, int p_cap, int32_t *a_idx, int32_t *a_cnt,
                       int a_cap, int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap, hipStream_t stream) {
    TopkParams tp = {};
    tp.m_pages = m_pages;
    tp.page_table = kv.page_table;
    tp.max_pages = kv.max_pages;
    tp.scores = scores;
    tp.seq_len = kv.seq_len;
    tp.p_idx = p_idx;
    tp.p_cnt = p_cnt;
    tp.a_idx = a_idx;
    tp.a_cnt = a_cnt;
    tp.m_idx = m_idx;
    tp.m_cnt = m_cnt;
    tp.hkv = kv.hkv;
    tp.block = block;
    tp.nmax = nmax;
    tp.topk = topk;
    tp.p_cap = p_cap;
    tp.a_cap = a_cap;
    tp.m_cap = m_cap;
    return dispatch_topk<TopkLaunch>(nmax, kv.batch * kv.hkv, tp, stream);
}

hipError_t launch_topk_groups(const KvDesc &kv, int block, int nmax, int topk, const int32_t *p_idx,
                              const int32_t *p_cnt, int p_cap, int32_t *a_idx, int32_t *a_cnt, int32_t *a_pages,
                              int a_cap, int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap,
                              const SelectSpecPlan &plan, int nparts, void *cand1, void *cand2, uint32_t *arrivals,
                              hipStream_t stream, int32_t *live) {
    TopkParams tp = {};
    tp.a_pages = a_pages;
    tp.m_pages = m_pages;
    tp.page_table = kv.page_table;
    tp.max_pages = kv.max_pages;
    tp.seq_len = kv.seq_len;
    tp.p_idx = p_idx;
    tp.p_cnt = p_cnt;
    tp.a_idx = a_idx;
    tp.a_cnt = a_cnt;
    tp.m_idx = m_idx;
    tp.m_cnt = m_cnt;
    tp.hkv = kv.hkv;
    tp.block = block;
    tp.nmax = nmax;
    tp.topk = topk;
    tp.p_cap = p_cap;
    tp.a_cap = a_cap;
    tp.m_cap = m_cap;
    const int units = kv.batch * kv.hkv;
    const size_t s1 = (size_t)units * nparts * plan.kl, s2 = (size_t)units * plan.ng * plan.kl2;
    CandParams c1, c2;
    c1.key = (uint64_t *)cand1;
    c1.idx = (int32_t *)((char *)cand1 + s1 * 8);
    c1.cnt = (int32_t *)((char *)cand1 + s1 * 12);
    c1.kl = plan.kl;
    c2.key = (uint64_t *)cand2;
    c2.idx = (int32_t *)((char *)cand2 + s2 * 8);
    c2.cnt = (int32_t *)((char *)cand2 + s2 * 12);
    c2.kl = plan.kl2;
    const dim3 grid(plan.ng, units);
#define PRR_TG(K2, K3)                                                                                      \
    if (plan.kpt2 == K2 && plan.kpt3 == K3) {                                                               \
        PRR_LAUNCH(topk_groups_kernel<K2, K3>, dim3(grid), dim3(256), stream, tp, c1, c2, arrivals, nparts, plan.gp, plan.ng, live); \
        return hipGetLastError();                                                                           \
    }
    PRR_TG(8, 1) PRR_TG(8, 2) PRR_TG(8, 4) PRR_TG(8, 8) PRR_TG(8, 16)
    PRR_TG(16, 1) PRR_TG(16, 2) PRR_TG(16, 4) PRR_TG(16, 8) PRR_TG(16, 16)
#undef PRR_TG
    return hipErrorInvalidValue;
}

// Part-parallel predictor shape for rows of nmax blocks: parts of 512 blocks, kl = min(budget, 512)
// candidates each, ranked with kpt slots per thread (two stages), or (kpt = 0, groups.three) through
// groups of parts first (three stages); neither: one workgroup per unit.
struct PredictPlan {
    int nparts, kl, kpt;
    SelectSpecPlan groups;
};

static PredictPlan predict_plan(int nmax, int budget) {
    PredictPlan pl = {};
    if (nmax <= 2048 || budget <= 0) return pl;   // one workgroup per unit holds the whole row
    pl.nparts = (nmax + 511) / 512;
    pl.kl = std::min(budget, 512);
    const long slots = (long)pl.nparts * pl.kl;
    pl.kpt = slots <= 1024 ? 4 : slots <= 2048 ? 8 : slots <= 4096 ? 16 : 0;
    if (pl.kpt == 0 && pl.nparts <= 256) {
        // three stages, as the selection's: groups of parts (up to 2048 candidate slots) keep their
        // top-|P|, then one ranking of the groups' candidates (up to 4096 slots)
        SelectSpecPlan &g = pl.groups;
        g.kl = pl.kl;
        g.gp = std::max(1, 2048 / pl.kl);
        if ((long)((pl.nparts + g.gp - 1) / g.gp) * std::min(budget, g.gp * pl.kl) > 4096)
            g.gp = std::max(1, 4096 / pl.kl);   // groups of up to 4096 slots leave fewer candidates to rank
        g.ng = (pl.nparts + g.gp - 1) / g.gp;
        g.kl2 = std::min(budget, g.gp * pl.kl);
        const long s2 = (long)std::min(g.gp, pl.nparts) * pl.kl, s3 = (long)g.ng * g.kl2;
        g.kpt2 = s2 <= 2048 ? 8 : 16;
        g.kpt3 = s3 <= 256 ? 1 : s3 <= 512 ? 2 : s3 <= 1024 ? 4 : s3 <= 2048 ? 8 : s3 <= 4096 ? 16 : 0;
        g.three = g.kpt3 != 0;
    }
    if (pl.nparts > 256 || (pl.kpt == 0 && !pl.groups.three)) pl = PredictPlan{};
    return pl;
}

size_t predict_workspace_bytes(int batch, int hkv, int nmax, int budget) {
    const PredictPlan pl = predict_plan(nmax, budget);
    if (pl.kpt == 0 && !pl.groups.three) return 0;
    const size_t units = (size_t)batch * hkv;
    const size_t parts = units * pl.nparts;
    size_t bytes = (units * 4 + 255) / 256 * 256 + parts * pl.kl * 12 + parts * 4;
    if (pl.groups.three) {
        const size_t groups = units * pl.groups.ng;
        bytes = (bytes + 255) / 256 * 256 + groups * pl.groups.kl2 * 12 + groups * 4;
    }
    return bytes;
}

hipError_t launch_predict(const double *scores, const int32_t *seq_len, int batch, int hkv,
                          int block, int nmax, double alpha, double beta, double gamma, int budget,
                          double *level, double *trend, int32_t *live, int32_t *p_idx,
                          int32_t *p_cnt, int32_t *p_pages, int p_cap, const int32_t *page_table, int max_pages,
                          void *ws, hipStream_t stream) {
    PredictParams p = {};
    p.p_pages = p_pages;
    p.page_table = page_table;
    p.max_pages = max_pages;
    p.scores = scores;
    p.seq_len = seq_len;
    p.level = level;
    p.trend = trend;
    p.live = live;
    p.p_idx = p_idx;
    p.p_cnt = p_cnt;
    p.hkv = hkv;
    p.block = block;
    p.nmax = nmax;
    p.budget = budget;
    p.p_cap = p_cap;
    p.alpha = alpha;
    p.beta = beta;
    p.gamma = gamma;
    const int units = batch * hkv;
    const PredictPlan pl = predict_plan(nmax, budget);
    if (!ws || (pl.kpt == 0 && !pl.groups.three)) return dispatch_topk<PredictLaunch>(nmax, units, p, stream);
    TopkParams tp = {};
    tp.seq_len = seq_len;
    tp.a_idx = p_idx;
    tp.a_cnt = p_cnt;
    tp.a_pages = p_pages;
    tp.page_table = page_table;
    tp.max_pages = max_pages;
    tp.m_idx = nullptr;   // no set difference
    tp.hkv = hkv;
    tp.block = block;
    tp.nmax = nmax;
    tp.topk = budget;
    tp.a_cap = p_cap;
    uint32_t *arrivals = (uint32_t *)ws;
    char *cbase = (char *)ws + ((size_t)units * 4 + 255) / 256 * 256;
    const size_t slots = (size_t)units * pl.nparts * pl.kl;
    CandParams cp;
    cp.key = (uint64_t *)cbase;
    cp.idx = (int32_t *)(cbase + slots * 8);
    cp.cnt = (int32_t *)(cbase + slots * 12);
    cp.kl = pl.kl;
    const dim3 grid(pl.nparts, units);
    if (pl.groups.three) {
        PRR_LAUNCH(predict_parts_only_kernel, dim3(grid), dim3(256), stream, p, cp, pl.nparts);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const size_t s1bytes = slots * 12 + (size_t)units * pl.nparts * 4;
        char *cand2 = cbase + (s1bytes + 255) / 256 * 256;
        KvDesc kv = {};
        kv.seq_len = seq_len;
        kv.page_table = page_table;
        kv.max_pages = max_pages;
        kv.batch = batch;
        kv.hkv = hkv;
        return launch_topk_groups(kv, block, nmax, budget, nullptr, nullptr, 0, p_idx, p_cnt, p_pages, p_cap, nullptr,
                                  nullptr, nullptr, 0, pl.groups, pl.nparts, cbase, cand2, arrivals, stream, live);
    }
    if (pl.kpt == 4) PRR_LAUNCH(predict_parts_kernel<4>, dim3(grid), dim3(256), stream, p, tp, cp, arrivals, pl.nparts);
    else if (pl.kpt == 8) PRR_LAUNCH(predict_parts_kernel<8>, dim3(grid), dim3(256), stream, p, tp, cp, arrivals, pl.nparts);
    else PRR_LAUNCH(predict_parts_kernel<16>, dim3(grid), dim3(256), stream, p, tp, cp, arrivals, pl.nparts);
    return hipGetLastError();
}

}  // namespace prr
