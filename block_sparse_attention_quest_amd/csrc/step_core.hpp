// step_core.hpp - selection and the speculative pass over P as one launch (gfx950).
//
// Citations:
//   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
//           Decoding" (full paper text)
//
// The method overlaps the speculative pass over the predicted set P with selection ([paper] §1 and the
// Figure 1 flow, §3): the two only read P and are independent.  On this GPU a dependency between two
// streams costs about 10 us from the producer's end to the consumer's start, while kernels on one
// stream follow each other about 1 us apart, so the overlap is made inside one grid instead: the first
// workgroups score blocks (one workgroup per 512 blocks of a unit, two per lane, for min/max metadata and
// for block means alike; 1024 blocks, four per lane, for the min/max metadata of rows of 32768 blocks and
// more that rank in three stages and of launches with more than 256 such parts), the rest run the
// speculative chunks (the attention kernels' chunk walk over
// n_spec workgroups, on bf16 or fp8 tiles: KT).  Dispatch follows the workgroup index, so
// the scoring workgroups issue their loads first: the memory system serves them ahead of the
// speculative stream, selection finishes early and its top-K runs under the speculative pass, which is
// the longer of the two.  At 128K, batch 8 the grid is 256 scoring + 256 speculative workgroups: all of
// them resident at once (two per CU).
//
// Top-K (with M = A \ P).  The last scoring workgroup of a unit to finish (a device-scope arrival
// counter; nobody waits) runs the unit's top-K with the same 256 threads, so the top-K of most units
// overlaps the speculative pass:
//   * up to 1024 blocks per unit, over all of the unit's scores (up to 4 per thread), stored and re-read
//     with device-scope accesses, which are coherent across the XCDs' L2s;
//   * beyond that, in two stages: every scoring workgroup first keeps the local top-min(K, part) of its
//     own part's blocks as candidates (in parallel, right after scoring), and the last one ranks the
//     candidates of all workgroups of the unit (up to 16 per thread; the selection is exact, see
//     select_core.hpp).  At 2048 blocks and K = 64 the last workgroup ranks 256 candidates instead of
//     2048 scores;
//   * with more candidates than one ranking holds, in three stages: the last part of each group of parts
//     keeps the group's top-K and the unit's last group ranks the groups' candidates (K2, K3 below), as
//     long as all scoring workgroups are resident at once; otherwise the launch keeps the parts'
//     candidates and the groups kernel follows it.
//
// Predictor step of another layer.  In a stack of layers the predictor of layer l needs only layer l's
// scores and is off the critical path ([paper] §1, §4.1), so layer l + 1's launch can carry it.  The
// scoring workgroups take its units from a work counter once their own scoring is done (and the top-K,
// for a unit's last arriver): the ones that finish first take most of them, the speculative pass keeps
// every slot it had (extra workgroups at the end of the grid would wait for a free slot and run past
// it), and the top-K is not delayed.  The two touch disjoint buffers.

#pragma once

#include "select_core.hpp"
#include "attn_core.hpp"

namespace prr {
namespace {

// Workgroup s < nsx * units scores blocks [BPW (s mod nsx), +BPW) of unit s / nsx (BPW = 512 blocks, two
// per lane, for bf16 min/max metadata and for fp32 block means: MEAN; 1024, four per lane, for the bf16
// min/max parts of long rows and of many-part launches: WIDE) and, if it is the unit's last to finish and
// KPT > 0, runs the unit's top-K (KPT keys per thread, 256 KPT >= the unit's block count); the remaining
// n_spec workgroups run the speculative pass.  PRED: the scoring workgroups then draw the n_pred units
// of another layer's predictor step from *pred_ctr (8 keys per thread: rows of up to 2048 blocks); every
// workgroup draws until it gets an index >= n_pred, so the launch makes exactly n_pred + n_score draws
// and the one that draws the last index resets the counter for the next launch.  Register use is the
// attention part's (two waves per SIMD).
//
// REP (the layer step as one launch): n_rep repair slots follow the speculative workgroups, every unit's
// speculative chunks and repair slots end in one merge over P u M (attn_core.hpp: FusedParams), and the
// top-K stores M with device-scope stores and then raises the unit's flag the repair slots wait for.
// K2, K3 (non-zero with TWO and KPT = 0): the three-stage top-K runs inside the launch too.  The last part
// of a group to arrive keeps the group's top-K (K2 candidate slots per thread), and the last group of a
// unit ranks the groups' candidates (K3 slots per thread) into A and M.
template <int KT, int D, int KPT, bool TWO, bool MEAN, bool PRED, bool REP = false, int K2 = 0, int K3 = 0,
          bool WIDE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void select_spec_kernel(
    AttnParams ap, ScoreParams sp, TopkParams tp, CandParams cp, GroupParams gq, PredictParams pp,
    uint32_t *arrivals, uint32_t *pred_ctr, int n_score, int nsx, int n_spec, int n_pred, FusedParams fp, int n_rep) {
    if ((int)blockIdx.x >= n_score) {
        if constexpr (REP) {
            __shared__ AttnSmem<D> asm_;
            const int w = (int)blockIdx.x - n_score;
            if (w < n_spec) attn_chunks<KT, D, false, 1, true>(ap, fp, w, n_spec, asm_);
            else fused_repair_slots<KT, D, 2>(ap, fp, w - n_spec, n_rep, asm_);
        } else {
            attn_body<KT, D, false, 1>(ap, (int)blockIdx.x - n_score, n_spec);
        }
        return;
    }
    const int s = (int)blockIdx.x;
    const int u = s / nsx;
    const int bx = s - u * nsx;
    static_assert(!WIDE || (TWO && !MEAN), "wide scoring parts: bf16 min/max rows of a staged top-K");
    constexpr int BPL = WIDE ? kWideScoreBPL : kScoreBPL<true, MEAN>;
    double kept[BPL] = {};
    score_body<true, D, KPT != 0 && !TWO, MEAN, BPL>(sp, bx, u, kept);
    if constexpr (TWO) {
        __shared__ TopkSmem<4> sm;
        constexpr int BPW = 256 * BPL;   // blocks per scoring workgroup
        const int b = u / sp.hkv;
        const int nb = min((max(sp.seq_len[b], 0) + sp.block - 1) / sp.block, sp.nmax);
        const int n_local = min(max(nb - bx * BPW, 0), BPW);
        const size_t part = (size_t)u * nsx + bx;
        local_candidates<BPL>(kept, n_local, cp.kl, bx * BPW, cp.key + part * cp.kl, cp.idx + part * cp.kl,
                              cp.cnt + part, sm);
    }
    if constexpr (K2 != 0) {
        static_assert(TWO && KPT == 0, "the in-launch groups follow part-local candidates");
        __shared__ int s_last_part, s_last_group;
        const int g = bx / gq.gp, p0 = g * gq.gp;
        const int gparts = min(gq.gp, nsx - p0);
        // this part's candidate stores are complete before its arrival is counted
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        uint32_t *pa = &gq.part_arr[(size_t)u * gq.ng + g];
        if (threadIdx.x == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(pa, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last_part = prev == (uint32_t)(gparts - 1);
            if (s_last_part) __hip_atomic_store(pa, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (s_last_part) {
            const size_t in = (size_t)u * nsx + p0, out = (size_t)u * gq.ng + g;
            group_candidates<K2>(cp.key + in * cp.kl, cp.idx + in * cp.kl, cp.cnt + in, gparts, cp.kl, gq.c2.kl,
                                 gq.c2.key + out * gq.c2.kl, gq.c2.idx + out * gq.c2.kl, gq.c2.cnt + out);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (threadIdx.x == 0) {
                const uint32_t prev = __hip_atomic_fetch_add(&gq.group_arr[u], 1u, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                s_last_group = prev == (uint32_t)(gq.ng - 1);
                if (s_last_group) __hip_atomic_store(&gq.group_arr[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            if (s_last_group) {
                const size_t g0 = (size_t)u * gq.ng;
                topk_candidates_body<K3, REP, kMaxSelectN>(tp, u, gq.c2.key + g0 * gq.c2.kl, gq.c2.idx + g0 * gq.c2.kl,
                                                           gq.c2.cnt + g0, gq.ng, gq.c2.kl);
                if constexpr (REP) {
                    // M's device-scope stores are complete before the unit's repair slots may read it
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
                    if (threadIdx.x == 0) __hip_atomic_store(&fp.ready[u * kReadyStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
    if constexpr (KPT != 0) {
        __shared__ int s_last;
        // this workgroup's score stores are complete before its arrival is counted
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(&arrivals[u], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = prev == (uint32_t)(nsx - 1);
            if (s_last) __hip_atomic_store(&arrivals[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (s_last) {
            if constexpr (TWO)
                topk_candidates_body<KPT, REP>(tp, u, cp.key + (size_t)u * nsx * cp.kl,
                                               cp.idx + (size_t)u * nsx * cp.kl, cp.cnt + (size_t)u * nsx, nsx, cp.kl);
            else
                topk_body<KPT, 256, true, REP>(tp, u);
            if constexpr (REP) {
                // M's device-scope stores are complete before the unit's repair slots may read it
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (threadIdx.x == 0) __hip_atomic_store(&fp.ready[u * kReadyStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if constexpr (PRED) {
        __shared__ int s_j;
        for (;;) {
            __syncthreads();   // the workgroup's shared scratch is free again, s_j read by every thread
            if (threadIdx.x == 0) {
                const uint32_t j = __hip_atomic_fetch_add(pred_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (j == (uint32_t)(n_pred + n_score - 1))
                    __hip_atomic_store(pred_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_j = (int)j;
            }
            __syncthreads();
            const int j = s_j;
            if (j >= n_pred) break;
            predict_body<8, 256>(pp, j);
        }
    }
}


// Candidate slots per thread of a fused launch's in-launch groups (K2) and final ranking (K3), encoded
// as K2 * 100 + K3: the instantiated pairs (8, 4), (8, 8), (8, 16) and (16, 16) cover every plan, a
// ranking of fewer slots taking the next width up.  0: the stages do not run inside the launch (no three
// stages, or more scoring workgroups than are resident at once: a part that ran a group's stage would
// hold its slot while other parts wait for one).
inline int three_stage_kpt(const SelectSpecPlan &pl, long n_score_wgs) {
    if (!pl.three || n_score_wgs > 2L * device_cu_count()) return 0;
    const int k3 = pl.kpt3 <= 4 ? 4 : pl.kpt3;
    return pl.kpt2 <= 8 ? 800 + k3 : 1616;
}

// Everything a fused launch needs besides its kernel: the parameters of its roles, its grid, and where the
// top-K stages after it (if any) keep their candidates.  Shared by the selection + speculation launch and
// the layer-step launch (which adds the repair slots).
struct FusedSetup {
    AttnParams ap;
    ScoreParams sp;
    TopkParams tp;
    CandParams cp;
    GroupParams gq;   // the in-launch groups of a three-stage top-K (plan.three)
    int k23;          // three_stage_kpt: the in-launch stages' widths, 0 if they run after the launch
    PredictParams pp;
    SelectSpecPlan plan;
    uint32_t *arrivals;
    uint32_t *pred_ctr;
    char *cbase;
    int units, nsx, n_spec, n_pred;
    bool fuse_pred;
    long grid;   // scoring + speculative workgroups
};

inline FusedSetup fused_setup(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride, int nmax,
                              int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap, double *scores,
                              int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap,
                              float scale, float *acc, float *l, float *m, float *out, void *ws, bool mean,
                              const PredictArgs *pred) {
    FusedSetup f{};
    // Two workgroups of this kernel fit on a CU.  When the scoring workgroups take more than half of
    // those slots (rows longer than 512 blocks per CU's share, e.g. a cache with room for appended
    // tokens), the speculative pass is spread over the slots that are left, so that the whole grid is
    // resident from the start instead of speculative workgroups waiting for scoring ones to finish.
    const int cus = device_cu_count();
    f.plan = select_spec_plan(nmax, topk, mean, kv.batch * kv.hkv);
    const int bpw = f.plan.bpw;
    const int n_score_wgs = (nmax + bpw - 1) / bpw * kv.batch * kv.hkv;
    const int spec_target = n_score_wgs > cus ? std::max(cus / 2, 2 * cus - n_score_wgs) : cus;
    f.n_spec = attn_setup(f.ap, kv, q, hq, block, p_idx, p_cnt, p_pages, p_cap, scale, acc, l, m, out, false, ws, spec_target);
    ScoreParams &sp = f.sp;
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
    TopkParams &tp = f.tp;
    tp = TopkParams{};
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
    f.units = kv.batch * kv.hkv;
    f.arrivals = (uint32_t *)ws + f.units;   // the scoring-arrival counters of the workspace
    f.nsx = (nmax + bpw - 1) / bpw;
    // (a launch with wide scoring parts leaves a carried predictor to its own launch: no instantiation)
    f.fuse_pred = pred && pred->nmax <= kMaxFusedPredictN && f.plan.bpw != score_bpw(true, false, true);
    f.pp = PredictParams{};
    f.n_pred = 0;
    if (f.fuse_pred) {
        PredictParams &pp = f.pp;
        pp.scores = pred->scores;
        pp.seq_len = pred->seq_len;
        pp.level = pred->level;
        pp.trend = pred->trend;
        pp.live = pred->live;
        pp.p_idx = pred->p_idx;
        pp.p_cnt = pred->p_cnt;
        pp.hkv = pred->hkv;
        pp.block = pred->block;
        pp.nmax = pred->nmax;
        pp.budget = pred->budget;
        pp.p_cap = pred->p_cap;
        pp.alpha = pred->alpha;
        pp.beta = pred->beta;
        pp.gamma = pred->gamma;
        pp.p_pages = pred->p_pages;
        pp.page_table = pred->page_table;
        pp.max_pages = pred->max_pages;
        f.n_pred = pred->batch * pred->hkv;
    }
    f.grid = (long)f.n_spec + (long)f.nsx * f.units;
    f.pred_ctr = (uint32_t *)((char *)ws + pred_counter_offset(kv.batch, hq, kv.hkv, kv.d, block, p_cap, nmax, topk, false));
    f.cp.kl = f.plan.kl;
    f.cbase = (char *)ws + attn_workspace_bytes(kv.batch, hq, kv.hkv, kv.d, block, p_cap);
    f.cp.key = (uint64_t *)f.cbase;
    f.cp.idx = (int32_t *)(f.cbase + (size_t)f.units * f.nsx * f.plan.kl * 8);
    f.cp.cnt = (int32_t *)(f.cbase + (size_t)f.units * f.nsx * f.plan.kl * 12);
    f.gq = GroupParams{};
    f.k23 = three_stage_kpt(f.plan, (long)f.nsx * f.units);
    if (f.plan.three) {
        const StageLayout sl = stage_layout(f.cbase, f.units, f.nsx, f.plan);
        const size_t s2 = (size_t)f.units * f.plan.ng * f.plan.kl2;
        f.gq.c2.key = (uint64_t *)sl.cand2;
        f.gq.c2.idx = (int32_t *)(sl.cand2 + s2 * 8);
        f.gq.c2.cnt = (int32_t *)(sl.cand2 + s2 * 12);
        f.gq.c2.kl = f.plan.kl2;
        f.gq.part_arr = sl.parr;
        f.gq.group_arr = sl.garr;
        f.gq.gp = f.plan.gp;
        f.gq.ng = f.plan.ng;
    }
    return f;
}

// The top-K stages that follow a fused launch whose ranking does not finish inside it.
inline hipError_t fused_after(const FusedSetup &f, const KvDesc &kv, int block, int nmax, int topk, const double *scores,
                              const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap, int32_t *a_idx, int32_t *a_cnt,
                              int a_cap, int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap, hipStream_t stream) {
    if (f.plan.three) {
        if (f.k23) return hipSuccess;   // the groups and the ranking ran inside the launch
        // the parts' candidates are in place; groups of them, then the unit's ranking
        const StageLayout sl = stage_layout(f.cbase, f.units, f.nsx, f.plan);
        return launch_topk_groups(kv, block, nmax, topk, p_idx, p_cnt, p_cap, a_idx, a_cnt, nullptr, a_cap, m_idx, m_cnt,
                                  m_pages, m_cap, f.plan, f.nsx, sl.cand1, sl.cand2, sl.garr, stream);
    }
    if (f.plan.kpt == 0)
        return launch_topk(kv, block, nmax, topk, scores, p_idx, p_cnt, p_cap, a_idx, a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap,
                           stream);
    return hipSuccess;
}

inline hipError_t predict_alone(const PredictArgs *pred, hipStream_t stream) {
    if (!pred) return hipSuccess;
    return launch_predict(pred->scores, pred->seq_len, pred->batch, pred->hkv, pred->block, pred->nmax, pred->alpha,
                          pred->beta, pred->gamma, pred->budget, pred->level, pred->trend, pred->live, pred->p_idx,
                          pred->p_cnt, pred->p_pages, pred->p_cap, pred->page_table, pred->max_pages, pred->ws, stream);
}

// The fused launch for caches of element type KT (bf16 or fp8; an f32 cache runs the passes in turn).
template <int KT>
hipError_t launch_select_spec_t(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride,
                              int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap,
                              double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx,
                              int32_t *m_cnt, int32_t *m_pages, int m_cap, float scale, float *acc, float *l, float *m,
                              void *ws, bool mean, const PredictArgs *pred, hipStream_t stream) {
    if constexpr (KT == kKtF32) {
        // fp32 caches (exact-input checks): the passes one after the other
        hipError_t e = launch_select(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_cap, scores,
                                     a_idx, a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, mean,
                                     (char *)ws + attn_workspace_bytes(kv.batch, hq, kv.hkv, kv.d, block, p_cap), stream);
        if (e != hipSuccess) return e;
        e = launch_attn(kv, q, hq, block, p_idx, p_cnt, p_pages, p_cap, scale, acc, l, m, nullptr, false, ws, stream);
        if (e != hipSuccess) return e;
        return predict_alone(pred, stream);
    } else {
    const FusedSetup f = fused_setup(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores, a_idx,
                                     a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, nullptr, ws, mean, pred);
    if (f.grid > 0x7fffffffL) return hipErrorInvalidValue;
    const int kpt = f.plan.kpt;
    const bool two = f.plan.two;
    const int k23 = f.k23;
    const bool wide = f.plan.bpw == score_bpw(true, false, true);
    const FusedParams none{};
#define PRR_SSW(DD, K, T, MN, PR, K2, K3, W)                                                               \
    if (kv.d == DD && kpt == K && two == T && mean == MN && f.fuse_pred == PR && k23 == K2 * 100 + K3 &&   \
        wide == W) {                                                                                        \
        PRR_LAUNCH((select_spec_kernel<KT, DD, K, T, MN, PR, false, K2, K3, W>), dim3((int)f.grid), dim3(256), stream, \
                   f.ap, f.sp, f.tp, f.cp, f.gq, f.pp, f.arrivals, f.pred_ctr, f.nsx * f.units, f.nsx, f.n_spec,  \
                   f.n_pred, none, 0);                                                                      \
    } else
#define PRR_SS(DD, K, T, MN, PR, K2, K3) PRR_SSW(DD, K, T, MN, PR, K2, K3, false)
// wide scoring parts: bf16 min/max rows of two stages (2 to 16 slots per thread) or three; a carried
// predictor runs as its own launch
#define PRR_SS_WIDE(DD)                                                                                     \
    PRR_SSW(DD, 2, true, false, false, 0, 0, true) PRR_SSW(DD, 4, true, false, false, 0, 0, true)            \
    PRR_SSW(DD, 8, true, false, false, 0, 0, true) PRR_SSW(DD, 16, true, false, false, 0, 0, true)           \
    PRR_SSW(DD, 0, true, false, false, 0, 0, true) PRR_SSW(DD, 0, true, false, false, 8, 4, true)            \
    PRR_SSW(DD, 0, true, false, false, 8, 8, true) PRR_SSW(DD, 0, true, false, false, 8, 16, true)           \
    PRR_SSW(DD, 0, true, false, false, 16, 16, true)
#define PRR_SS_K(DD, MN, PR)                                                                                \
    PRR_SS(DD, 0, false, MN, PR, 0, 0) PRR_SS(DD, 0, true, MN, PR, 0, 0)                                     \
    PRR_SS(DD, 0, true, MN, PR, 8, 4) PRR_SS(DD, 0, true, MN, PR, 8, 8) PRR_SS(DD, 0, true, MN, PR, 8, 16)    \
    PRR_SS(DD, 0, true, MN, PR, 16, 16)                                                                     \
    PRR_SS(DD, 1, false, MN, PR, 0, 0) PRR_SS(DD, 2, false, MN, PR, 0, 0)                                          \
    PRR_SS(DD, 4, false, MN, PR, 0, 0) PRR_SS(DD, 8, false, MN, PR, 0, 0) PRR_SS(DD, 1, true, MN, PR, 0, 0)           \
    PRR_SS(DD, 2, true, MN, PR, 0, 0) PRR_SS(DD, 4, true, MN, PR, 0, 0) PRR_SS(DD, 8, true, MN, PR, 0, 0)             \
    PRR_SS(DD, 16, true, MN, PR, 0, 0)
#define PRR_SS_ALL(MN, PR) PRR_SS_K(128, MN, PR) PRR_SS_K(64, MN, PR)
    PRR_SS_WIDE(128) PRR_SS_WIDE(64)
    PRR_SS_ALL(false, false) PRR_SS_ALL(true, false) PRR_SS_ALL(false, true) PRR_SS_ALL(true, true)
    { return hipErrorInvalidValue; }
#undef PRR_SS_ALL
#undef PRR_SS_K
#undef PRR_SS_WIDE
#undef PRR_SS
#undef PRR_SSW
    hipError_t e = fused_after(f, kv, block, nmax, topk, scores, p_idx, p_cnt, p_pages, p_cap, a_idx, a_cnt, a_cap, m_idx, m_cnt,
                               m_pages, m_cap, stream);
    if (e != hipSuccess) return e;
    return f.fuse_pred ? hipSuccess : predict_alone(pred, stream);
    }
}

// Where the layer-step workspace keeps what prr_select_spec's does not have: M's attention workspace (for
// the repair chunks' partial states, or for prr_repair's own launch), then the per-unit M flags and the
// status word, each 256-byte aligned.
inline size_t layer_extra_m_ws(int batch, int hq, int hkv, int d, int block, int m_cap) {
    return attn_workspace_bytes(batch, hq, hkv, d, block, m_cap);
}

// The layer step (selection, the speculative pass over P, repair over M = A \ P) for caches of element
// type KT: one launch when the cache is bf16 or fp8 and the top-K finishes inside the launch (rows of up
// to 4096 candidate slots); otherwise prr_select_spec's launches followed by prr_repair's.  mws: the M
// part of the workspace (layer_extra_m_ws bytes, then the flags).
template <int KT>
hipError_t launch_layer_step_t(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride,
                               int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap,
                               double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx,
                               int32_t *m_cnt, int32_t *m_pages, int m_cap, float scale, float *acc, float *l, float *m, float *out,
                               void *ws, void *mws, bool mean, const PredictArgs *pred, hipStream_t stream) {
    const int units = kv.batch * kv.hkv;
    const size_t mbytes = layer_extra_m_ws(kv.batch, hq, kv.hkv, kv.d, block, m_cap);
    uint32_t *ready = (uint32_t *)((char *)mws + mbytes);
    uint32_t *status = (uint32_t *)((char *)mws + mbytes + (size_t)units * 4 * kReadyStride);
    const SelectSpecPlan plan = select_spec_plan(nmax, topk, mean, units);
    const int bpw = plan.bpw;
    const long n_score_wgs = (long)((nmax + bpw - 1) / bpw) * units;
    if (KT == kKtF32 || (plan.kpt == 0 && !plan.three) || (plan.three && three_stage_kpt(plan, n_score_wgs) == 0)) {
        hipError_t e = launch_select_spec(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores,
                                          a_idx, a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, ws, mean, pred,
                                          stream);
        if (e != hipSuccess) return e;
        return launch_attn(kv, q, hq, block, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, out, true, mws, stream);
    } else {
    const FusedSetup f = fused_setup(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores, a_idx,
                                     a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, out, ws, mean, pred);
    FusedParams fp{};
    attn_setup(fp.pm, kv, q, hq, block, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, out, true, mws);
    // M's chunks at half prr_repair's size (at least kChunkMin pages; the workspace's partial slots are
    // counted at kChunkStep): the repair slots start only once their unit's top-K is done, late in the
    // launch, so more and shorter chunks finish sooner
    fp.pm.cp = std::max(kChunkMin, (fp.pm.cp / 2 + kChunkStep - 1) / kChunkStep * kChunkStep);
    fp.pm.kmax = std::max(1, (m_cap * (block / kPage) + fp.pm.cp - 1) / fp.pm.cp);
    fp.ready = ready;
    fp.status = status;
    const long n_rep = (long)units * fp.pm.kmax;
    const long grid = f.grid + n_rep;
    if (grid > 0x7fffffffL) return hipErrorInvalidValue;
    const int kpt = plan.kpt;
    const bool two = plan.two;
    const int k23 = f.k23;
    const bool wide = plan.bpw == score_bpw(true, false, true);
#define PRR_LSW(DD, K, T, MN, PR, K2, K3, W)                                                               \
    if (kv.d == DD && kpt == K && two == T && mean == MN && f.fuse_pred == PR && k23 == K2 * 100 + K3 &&   \
        wide == W) {                                                                                        \
        PRR_LAUNCH((select_spec_kernel<KT, DD, K, T, MN, PR, true, K2, K3, W>), dim3((int)grid), dim3(256), stream, \
                   f.ap, f.sp, f.tp, f.cp, f.gq, f.pp, f.arrivals, f.pred_ctr, f.nsx * f.units, f.nsx, f.n_spec,  \
                   f.n_pred, fp, (int)n_rep);                                                               \
    } else
#define PRR_LS(DD, K, T, MN, PR, K2, K3) PRR_LSW(DD, K, T, MN, PR, K2, K3, false)
#define PRR_LS_WIDE(DD)                                                                                     \
    PRR_LSW(DD, 2, true, false, false, 0, 0, true) PRR_LSW(DD, 4, true, false, false, 0, 0, true)            \
    PRR_LSW(DD, 8, true, false, false, 0, 0, true) PRR_LSW(DD, 16, true, false, false, 0, 0, true)           \
    PRR_LSW(DD, 0, true, false, false, 8, 4, true) PRR_LSW(DD, 0, true, false, false, 8, 8, true)            \
    PRR_LSW(DD, 0, true, false, false, 8, 16, true) PRR_LSW(DD, 0, true, false, false, 16, 16, true)
#define PRR_LS_K(DD, MN, PR)                                                                                \
    PRR_LS(DD, 1, false, MN, PR, 0, 0) PRR_LS(DD, 2, false, MN, PR, 0, 0) PRR_LS(DD, 4, false, MN, PR, 0, 0)  \
    PRR_LS(DD, 1, true, MN, PR, 0, 0) PRR_LS(DD, 2, true, MN, PR, 0, 0) PRR_LS(DD, 4, true, MN, PR, 0, 0)     \
    PRR_LS(DD, 8, true, MN, PR, 0, 0) PRR_LS(DD, 16, true, MN, PR, 0, 0)                                    \
    PRR_LS(DD, 0, true, MN, PR, 8, 4) PRR_LS(DD, 0, true, MN, PR, 8, 8) PRR_LS(DD, 0, true, MN, PR, 8, 16)    \
    PRR_LS(DD, 0, true, MN, PR, 16, 16)
#define PRR_LS_ALL(MN, PR) PRR_LS_K(128, MN, PR) PRR_LS_K(64, MN, PR)
    PRR_LS_WIDE(128) PRR_LS_WIDE(64)
    PRR_LS_ALL(false, false) PRR_LS_ALL(true, false) PRR_LS_ALL(false, true) PRR_LS_ALL(true, true)
    { return hipErrorInvalidValue; }
#undef PRR_LS_ALL
#undef PRR_LS_K
#undef PRR_LS_WIDE
#undef PRR_LS
#undef PRR_LSW
    return f.fuse_pred ? hipSuccess : predict_alone(pred, stream);
    }
}

}  // namespace
}  // namespace prr
