// step.hip - the fused selection + speculation launch for bf16 caches, its plan and workspace (gfx950).
// The device code and its design notes are in step_core.hpp; fp8 caches are instantiated in
// step_fp8.hip.

#include "step_core.hpp"

namespace prr {


// Rows of up to 1024 blocks are ranked in one stage; longer rows in two (part-local candidates, then the
// candidates of all parts).  At 2048 blocks (128K context, block 64, batch 8) two stages took the fused
// launch from 37.2 to 35.4 us: the candidate selection runs in every scoring workgroup in parallel, and
// the unit's last workgroup ranks 256 candidates instead of 2048 scores.
SelectSpecPlan stage_plan(int nmax, int topk, int bpw, bool force_three) {
    SelectSpecPlan pl = {};
    pl.bpw = bpw;
    pl.two = false;
    pl.kl = 0;
    pl.kpt = force_three ? 0 : nmax <= 256 ? 1 : nmax <= 512 ? 2 : nmax <= 1024 ? 4 : 0;
    if (pl.kpt == 0 && nmax <= kMaxSelectN) {
        const int nsx = (nmax + bpw - 1) / bpw;
        const int kl = std::max(1, std::min(topk, bpw));
        const long slots = (long)nsx * kl;
        const int kpt = slots <= 256 ? 1 : slots <= 512 ? 2 : slots <= 1024 ? 4 : slots <= 2048 ? 8
                      : slots <= 4096 ? 16 : 0;
        if (kpt && !force_three) {
            pl.two = true;
            pl.kl = kl;
            pl.kpt = kpt;
        } else {
            // three stages: groups of parts with up to 2048 candidate slots keep their top-K each, and
            // one ranking of the groups' candidates (up to 4096 slots) follows.  At 32768 blocks and
            // K = 256 (8 groups of 8 parts) this took the 512K layer step from 96.9 to 73.6 us; groups of
            // 4096 slots (4 per unit, fewer workgroups) took 76.7 us, so they are used only where groups
            // of 2048 slots would leave more than one ranking holds (K above 341 at 32768 blocks).  A
            // group is one workgroup of 256 threads, one part's count each: at most 256 parts.
            int gp = std::min(256, std::max(1, 2048 / kl));
            if ((long)((nsx + gp - 1) / gp) * std::min(topk, gp * kl) > 4096)
                gp = std::min(256, std::max(1, 4096 / kl));   // groups of up to 4096 slots: fewer candidates remain
            const int ng = (nsx + gp - 1) / gp;
            const int kl2 = std::min(topk, gp * kl);
            const long slots2 = (long)std::min(gp, nsx) * kl, slots3 = (long)ng * kl2;
            const int kpt2 = slots2 <= 2048 ? 8 : 16;
            const int kpt3 = slots3 <= 256 ? 1 : slots3 <= 512 ? 2 : slots3 <= 1024 ? 4 : slots3 <= 2048 ? 8
                           : slots3 <= 4096 ? 16 : 0;
            if (kpt3 && ng <= 256) {
                pl.two = true;
                pl.kl = kl;
                pl.kpt = 0;
                pl.three = true;
                pl.gp = gp;
                pl.ng = ng;
                pl.kl2 = kl2;
                pl.kpt2 = kpt2;
                pl.kpt3 = kpt3;
            }
        }
    }
    return pl;
}

// The fused launch ranks a unit in two stages only for rows whose P bitmap one ranking holds
// (kMaxTwoStageBlocks); longer rows take the three stages (inside the launch when its scoring workgroups
// are resident, else the last two in launches of their own).  Rows of kWideScoreBlocks and more score
// four blocks per lane where that plan takes three stages too.
// Wide parts also go to rows of more than kMaxFusedPredictN blocks (a carried predictor is never
// affected) whose 512-block parts would number more than kWideScoreParts over all units, where the plan
// at 1024 blocks ranks in two stages with 2 to 16 slots per thread or in three: at 256K, batch 4,
// G = 8 (8192 blocks, 512 parts) select_spec went from 47.3 to 40.9 us and the layer step from 59.8 to
// 53.5 us.  With fewer parts than CUs the narrow parts keep the chip busier (128K, batch 8: 256 parts).
SelectSpecPlan select_spec_plan(int nmax, int topk, bool mean, int units) {
    const bool force = nmax > kMaxTwoStageBlocks;
    if (!mean) {
        const bool long_row = nmax >= kWideScoreBlocks;
        const bool many_parts = nmax > kMaxFusedPredictN &&
                                (long)((nmax + score_bpw(true, false) - 1) / score_bpw(true, false)) * units > kWideScoreParts;
        if (long_row || many_parts) {
            const SelectSpecPlan wide = stage_plan(nmax, topk, score_bpw(true, false, true), force);
            if (wide.three || (many_parts && wide.two && wide.kpt >= 2)) return wide;
        }
    }
    return stage_plan(nmax, topk, score_bpw(true, mean), force);
}

SelectSpecPlan select_stage_plan(int nmax, int topk, bool bq, bool mean) {
    if (bq && !mean && nmax >= kWideScoreBlocks) {
        const SelectSpecPlan wide = stage_plan(nmax, topk, score_bpw(true, false, true), true);
        if (wide.three) return wide;
    }
    return stage_plan(nmax, topk, score_bpw(bq, mean), true);
}

// Candidate slots of the two-stage top-K: [units][nsx][kl] keys (8 bytes) and indices (4), [units][nsx]
// counts.  The workspace covers both block summaries.  A three-stage top-K appends the group candidates
// ([units][ng][kl2] keys and indices, [units][ng] counts) and one group arrival counter per unit.
static size_t candidate_bytes(int units, int nmax, int topk, bool mean) {
    const SelectSpecPlan pl = select_spec_plan(nmax, topk, mean, units);
    if (!pl.two) return 0;
    const int nparts = (nmax + pl.bpw - 1) / pl.bpw;
    if (pl.three) return stage_layout(nullptr, units, nparts, pl).bytes;
    const size_t parts = (size_t)units * nparts;
    return parts * pl.kl * 12 + parts * 4;
}

size_t select_workspace_bytes(int units, int nmax, int topk, bool bq, bool mean) {
    if (nmax <= kStagedSelectMin) return 0;
    const SelectSpecPlan pl = select_stage_plan(nmax, topk, bq, mean);
    return pl.three ? stage_layout(nullptr, units, (nmax + pl.bpw - 1) / pl.bpw, pl).bytes : 0;
}

bool select_supported(int nmax, int topk, bool bq, bool mean) {
    return nmax <= kMaxRowTopK || (nmax <= kMaxSelectN && select_stage_plan(nmax, topk, bq, mean).three);
}

// The carried predictor's work counter sits after the candidates, in a 256-byte slot of its own.  For an
// fp32 cache, whose passes run in turn, the candidate room is launch_select's workspace instead.
size_t pred_counter_offset(int batch, int hq, int hkv, int d, int block, int cap, int nmax, int topk, bool f32) {
    const int units = batch * hkv;
    const size_t cand = f32 ? std::max(select_workspace_bytes(units, nmax, topk, false, false),
                                       select_workspace_bytes(units, nmax, topk, false, true))
                            : std::max(candidate_bytes(units, nmax, topk, false), candidate_bytes(units, nmax, topk, true));
    return attn_workspace_bytes(batch, hq, hkv, d, block, cap) + (cand + 255) / 256 * 256;
}

size_t select_spec_workspace_bytes(int batch, int hq, int hkv, int d, int block, int cap, int nmax, int topk, bool f32) {
    return pred_counter_offset(batch, hq, hkv, d, block, cap, nmax, topk, f32) + 256;
}

hipError_t launch_select_spec(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride,
                              int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap,
                              double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx,
                              int32_t *m_cnt, int32_t *m_pages, int m_cap, float scale, float *acc, float *l, float *m,
                              void *ws, bool mean, const PredictArgs *pred, hipStream_t stream) {
    if (kv.fp8)
        return launch_select_spec_fp8(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores,
                                      a_idx, a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, ws, mean, pred,
                                      stream);
    if (kv.bf16)
        return launch_select_spec_t<kKtBf16>(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap,
                                             scores, a_idx, a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m,
                                             ws, mean, pred, stream);
    return launch_select_spec_t<kKtF32>(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores,
                                        a_idx, a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, ws, mean,
                                        pred, stream);
}

}  // namespace prr
