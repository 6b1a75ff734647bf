// prr_api.cpp - the extern "C" boundary of libprr.so: argument validation, sizes, dispatch.
// Every check here runs before anything is enqueued; see include/prr.h for the contract.

#include "prr.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>

#include "prr_internal.hpp"

namespace {

// Kernel timing (prr_time_next_kernel).  The armed events move to the next entry-point call of the thread
// (the outermost one, when an entry point calls another): its first launch takes the start event and
// every launch the stop event; the call consumes them whether or not it launches.
struct TimingEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
thread_local TimingEvents t_armed;
thread_local TimingEvents t_call;
thread_local int t_depth = 0;

struct CallTiming {
    CallTiming() {
        if (t_depth++ == 0) {
            t_call = t_armed;
            t_armed = TimingEvents{};
        }
    }
    ~CallTiming() {
        if (--t_depth == 0) t_call = TimingEvents{};
    }
    CallTiming(const CallTiming &) = delete;
    CallTiming &operator=(const CallTiming &) = delete;
};

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

prr_status check_kv(const prr_kv_cache *kv) {
    if (!kv || !kv->k || !kv->v || !kv->page_table || !kv->seq_len) return PRR_EINVAL;
    if (kv->batch <= 0 || kv->num_kv_heads <= 0 || kv->num_pages <= 0 || kv->max_pages <= 0)
        return PRR_EINVAL;
    if (kv->page_size != prr::kPage) return PRR_EUNSUPPORTED;
    if (kv->head_dim != 64 && kv->head_dim != 128) return PRR_EUNSUPPORTED;
    if (kv->dtype != PRR_F32 && kv->dtype != PRR_BF16 && kv->dtype != PRR_FP8) return PRR_EUNSUPPORTED;
    return PRR_OK;
}

prr_status check_block(const prr_kv_cache *kv, int32_t block) {
    if (block <= 0 || block % kv->page_size != 0) return PRR_EINVAL;
    if ((int64_t)kv->max_pages * kv->page_size % block != 0) return PRR_EINVAL;
    return PRR_OK;
}

prr_status check_heads(const prr_kv_cache *kv, int32_t hq) {
    if (hq <= 0 || hq % kv->num_kv_heads != 0) return PRR_EINVAL;
    const int G = hq / kv->num_kv_heads;
    if (!is_pow2(G) || G > 16) return PRR_EUNSUPPORTED;
    return PRR_OK;
}

prr_status check_set(const prr_block_set *s) {
    if (!s || !s->idx || !s->count || s->cap <= 0) return PRR_EINVAL;
    return PRR_OK;
}

prr::KvDesc desc(const prr_kv_cache *kv) {
    prr::KvDesc d;
    d.k = kv->k;
    d.v = kv->v;
    d.page_table = kv->page_table;
    d.seq_len = kv->seq_len;
    d.batch = kv->batch;
    d.hkv = kv->num_kv_heads;
    d.d = kv->head_dim;
    d.num_pages = kv->num_pages;
    d.max_pages = kv->max_pages;
    d.bf16 = kv->dtype == PRR_BF16;
    d.fp8 = kv->dtype == PRR_FP8;
    return d;
}

prr_status hip_status(hipError_t e) { return e == hipSuccess ? PRR_OK : PRR_EHIP; }

// Checking mode: an input set's device-side preconditions (entries in range, no repeats).
prr_status check_input_set(const prr_kv_cache *kv, int32_t block, const prr_block_set *s, hipStream_t stream) {
    if (!s || !prr::checks_enabled()) return PRR_OK;
    int violation = 0;
    const hipError_t e = prr::check_sets(desc(kv), block, s->idx, s->count, s->cap, stream, &violation);
    if (e != hipSuccess) return PRR_EHIP;
    return violation ? PRR_EINVAL : PRR_OK;
}

#define PRR_TRY(x)                      \
    do {                                \
        const prr_status s_ = (x);      \
        if (s_ != PRR_OK) return s_;    \
    } while (0)

prr_status attn_common(const void *q, int32_t hq, const prr_kv_cache *kv, int32_t block,
                       const prr_block_set *set, void *ws, size_t ws_bytes) {
    if (!q) return PRR_EINVAL;
    PRR_TRY(check_kv(kv));
    PRR_TRY(check_block(kv, block));
    PRR_TRY(check_heads(kv, hq));
    PRR_TRY(check_set(set));
    const size_t need = prr::attn_workspace_bytes(kv->batch, hq, kv->num_kv_heads, kv->head_dim, block,
                                                  set->cap);
    if (!ws || ws_bytes < need) return PRR_EWORKSPACE;
    return PRR_OK;
}

}  // namespace

namespace prr {
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool take_kernel_timing(hipEvent_t *start, hipEvent_t *stop) {
    if (!t_call.start && !t_call.stop) return false;
    *start = t_call.start;   // the call's first kernel only
    *stop = t_call.stop;     // every kernel of the call, so the last one's end remains
    t_call.start = nullptr;
    return true;
}
}  // namespace prr

extern "C" {

prr_status prr_time_next_kernel(hipEvent_t start, hipEvent_t stop) {
    t_armed.start = start;
    t_armed.stop = stop;
    return PRR_OK;
}

int32_t prr_max_blocks(const prr_kv_cache *kv, int32_t block) {
    if (!kv || block <= 0) return 0;
    return (int32_t)((int64_t)kv->max_pages * kv->page_size / block);
}

int32_t prr_meta_stride(const prr_kv_cache *kv, int32_t block) {
    const int32_t n = prr_max_blocks(kv, block);
    return (n + 7) / 8 * 8;
}

size_t prr_meta_bytes(const prr_kv_cache *kv, int32_t block) {
    if (!kv) return 0;
    const size_t elem = kv->dtype == PRR_F32 ? 4 : 2;   // bf16 for bf16 and fp8 caches
    return (size_t)kv->batch * kv->num_kv_heads * kv->head_dim * 2 * prr_meta_stride(kv, block) * elem;
}

size_t prr_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block, int32_t cap) {
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block < prr::kPage ||
        cap <= 0)
        return 0;
    return prr::attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, block, cap);
}

prr_status prr_workspace_clear(void *ws, size_t ws_bytes, hipStream_t stream) {
    CallTiming timing_;
    if (!ws && ws_bytes) return PRR_EINVAL;
    return hip_status(prr::launch_clear(ws, ws_bytes, stream));
}

prr_status prr_build_meta(const prr_kv_cache *kv, int32_t block, void *meta, hipStream_t stream) {
    CallTiming timing_;
    PRR_TRY(check_kv(kv));
    PRR_TRY(check_block(kv, block));
    if (!meta) return PRR_EINVAL;
    return hip_status(prr::launch_meta(desc(kv), block, prr_meta_stride(kv, block), meta, false, stream));
}

size_t prr_mean_meta_bytes(const prr_kv_cache *kv, int32_t block) {
    if (!kv) return 0;
    return (size_t)kv->batch * kv->num_kv_heads * kv->head_dim * prr_meta_stride(kv, block) * sizeof(float);
}

prr_status prr_build_mean_meta(const prr_kv_cache *kv, int32_t block, float *meta, hipStream_t stream) {
    CallTiming timing_;
    PRR_TRY(check_kv(kv));
    PRR_TRY(check_block(kv, block));
    if (!meta) return PRR_EINVAL;
    return hip_status(prr::launch_meta(desc(kv), block, prr_meta_stride(kv, block), meta, true, stream));
}

prr_status prr_append(const prr_kv_cache *kv, int32_t block, const void *k_new, const void *v_new, void *meta,
                      prr_score_mode mode, int32_t *seq_len, hipStream_t stream) {
    CallTiming timing_;
    PRR_TRY(check_kv(kv));
    PRR_TRY(check_block(kv, block));
    if (!k_new || !v_new || !meta || !seq_len) return PRR_EINVAL;
    if (mode != PRR_SCORE_QUEST && mode != PRR_SCORE_MEAN) return PRR_EINVAL;
    if (seq_len != kv->seq_len) return PRR_EINVAL;   // the cache's own length array is advanced
    return hip_status(prr::launch_append(desc(kv), const_cast<void *>(kv->k), const_cast<void *>(kv->v), seq_len,
                                         k_new, v_new, block, prr_meta_stride(kv, block), meta,
                                         mode == PRR_SCORE_MEAN, stream));
}

// Whether selection (of any entry point) has a top-K plan for rows of nmax blocks: one top-K workgroup
// per unit up to prr::kMaxRowTopK blocks, the three part-parallel stages beyond.
static bool selection_plan_exists(const prr_kv_cache *kv, int nmax, int topk, bool mean, bool fused) {
    if (nmax > prr::kMaxSelectN) return false;
    if (nmax <= prr::kMaxRowTopK) return true;
    const bool bq = kv->dtype != PRR_F32;
    if (fused && bq) return prr::select_spec_plan(nmax, topk, mean, kv->batch * kv->num_kv_heads).three;
    return prr::select_supported(nmax, topk, bq, mean);
}

size_t prr_select_workspace_bytes(const prr_kv_cache *kv, prr_score_mode mode, int32_t block, int32_t topk) {
    if (!kv || kv->batch <= 0 || kv->num_kv_heads <= 0 || block < prr::kPage || topk < 0) return 0;
    if (mode != PRR_SCORE_QUEST && mode != PRR_SCORE_MEAN) return 0;
    return prr::select_workspace_bytes(kv->batch * kv->num_kv_heads, prr_max_blocks(kv, block), topk,
                                       kv->dtype != PRR_F32, mode == PRR_SCORE_MEAN);
}

prr_status prr_select(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, const void *meta,
                      prr_score_mode mode, int32_t block, int32_t topk, const prr_block_set *P, double *scores,
                      prr_block_set *A, prr_block_set *M, void *ws, size_t ws_bytes, hipStream_t stream) {
    CallTiming timing_;
    if (!q || !meta || !scores) return PRR_EINVAL;
    if (mode != PRR_SCORE_QUEST && mode != PRR_SCORE_MEAN) return PRR_EINVAL;
    PRR_TRY(check_kv(kv));
    PRR_TRY(check_block(kv, block));
    PRR_TRY(check_heads(kv, num_q_heads));
    PRR_TRY(check_set(A));
    if (topk < 0) return PRR_EINVAL;
    if (A->cap < topk) return PRR_EINVAL;
    if ((P == nullptr) != (M == nullptr)) return PRR_EINVAL;
    if (P) {
        PRR_TRY(check_set(P));
        PRR_TRY(check_set(M));
        if (M->cap < topk) return PRR_EINVAL;
    }
    const int nmax = prr_max_blocks(kv, block);
    if (!selection_plan_exists(kv, nmax, topk, mode == PRR_SCORE_MEAN, false)) return PRR_EUNSUPPORTED;
    // the stages' workspace: required above one top-K workgroup's rows, optional (faster) below
    const size_t need = prr_select_workspace_bytes(kv, mode, block, topk);
    if (nmax > prr::kMaxRowTopK && !ws) return PRR_EWORKSPACE;
    if (ws && ws_bytes < need) return PRR_EWORKSPACE;
    PRR_TRY(check_input_set(kv, block, P, stream));
    return hip_status(prr::launch_select(desc(kv), q, num_q_heads, meta, block, prr_meta_stride(kv, block),
                                         nmax, topk, P ? P->idx : nullptr, P ? P->count : nullptr,
                                         P ? P->cap : 0, scores, A->idx, A->count, A->cap,
                                         M ? M->idx : nullptr, M ? M->count : nullptr, M ? M->pages : nullptr,
                                         M ? M->cap : 0, mode == PRR_SCORE_MEAN, need ? ws : nullptr, stream));
}

size_t prr_select_spec_workspace_bytes(const prr_kv_cache *kv, int32_t num_q_heads, int32_t block, int32_t topk,
                                       int32_t cap) {
    if (!kv || kv->batch <= 0 || kv->num_kv_heads <= 0 || num_q_heads <= 0 || kv->head_dim <= 0 ||
        block < prr::kPage || cap <= 0 || topk < 0)
        return 0;
    return prr::select_spec_workspace_bytes(kv->batch, num_q_heads, kv->num_kv_heads, kv->head_dim, block, cap,
                                            prr_max_blocks(kv, block), topk, kv->dtype == PRR_F32);
}

static prr_status check_predict(const double *scores, const int32_t *seq_len, int32_t batch,
                                int32_t num_kv_heads, int32_t block, int32_t max_blocks, int32_t budget,
                                const double *level, const double *trend, const int32_t *live,
                                const prr_block_set *P_next, const prr_kv_cache *kv) {
    if (!scores || !seq_len || !level || !trend || !live) return PRR_EINVAL;
    if (batch <= 0 || num_kv_heads <= 0 || block <= 0 || max_blocks <= 0 || budget < 0) return PRR_EINVAL;
    PRR_TRY(check_set(P_next));
    if (P_next->cap < budget) return PRR_EINVAL;
    // rows longer than one workgroup's top-K need the part-parallel plan (and its workspace)
    if (max_blocks > prr::kMaxSelectN ||
        (max_blocks > prr::kMaxRowTopK && prr::predict_workspace_bytes(batch, num_kv_heads, max_blocks, budget) == 0))
        return PRR_EUNSUPPORTED;
    if (P_next->pages) {
        // the page list maps through this cache's page table, for the same sequences and block size
        PRR_TRY(check_kv(kv));
        PRR_TRY(check_block(kv, block));
        if (kv->batch != batch || kv->num_kv_heads != num_kv_heads) return PRR_EINVAL;
    }
    return PRR_OK;
}

// The carried predictor step's arguments (prr_select_spec_predict, prr_layer_step): checked, and with no
// buffer shared with the selection's outputs or P.
static prr_status predict_args(const prr_predict_args *pred, const double *scores, const prr_block_set *P,
                               const prr_block_set *A, const prr_block_set *M, prr::PredictArgs &pa) {
    pa = prr::PredictArgs{};
    if (pred) {
        PRR_TRY(check_predict(pred->scores, pred->seq_len, pred->batch, pred->num_kv_heads, pred->block,
                              pred->max_blocks, pred->budget, pred->level, pred->trend, pred->live, pred->P_next,
                              pred->kv));
        // the predictor writes level, trend, live and P_next while the selection writes scores, A and M
        // and reads P: none of them may be shared
        const void *sel_bufs[] = {scores, P->idx, P->count, P->pages, A->idx, A->count, M->idx, M->count, M->pages};
        const void *pred_out[] = {pred->level, pred->trend, pred->live, pred->P_next->idx, pred->P_next->count,
                                  pred->P_next->pages};
        for (const void *x : pred_out)
            for (const void *y : sel_bufs)
                if (x && x == y) return PRR_EINVAL;
        if ((const void *)pred->scores == (const void *)scores) return PRR_EINVAL;
        pa.scores = pred->scores;
        pa.seq_len = pred->seq_len;
        pa.batch = pred->batch;
        pa.hkv = pred->num_kv_heads;
        pa.block = pred->block;
        pa.nmax = pred->max_blocks;
        pa.budget = pred->budget;
        pa.alpha = pred->alpha;
        pa.beta = pred->beta;
        pa.gamma = pred->gamma;
        pa.level = pred->level;
        pa.trend = pred->trend;
        pa.live = pred->live;
        pa.p_idx = pred->P_next->idx;
        pa.p_cnt = pred->P_next->count;
        pa.p_cap = pred->P_next->cap;
        if (pred->P_next->pages) {
            pa.p_pages = pred->P_next->pages;
            pa.page_table = pred->kv->page_table;
            pa.max_pages = pred->kv->max_pages;
        }
        const size_t need = prr::predict_workspace_bytes(pred->batch, pred->num_kv_heads, pred->max_blocks,
                                                         pred->budget);
        if (pred->ws && pred->ws_bytes < need) return PRR_EWORKSPACE;
        if (pred->max_blocks > prr::kMaxRowTopK && !pred->ws) return PRR_EWORKSPACE;
        pa.ws = need ? pred->ws : nullptr;
    }
    return PRR_OK;
}

prr_status prr_select_spec_predict(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, const void *meta,
                                   prr_score_mode mode, int32_t block, int32_t topk, const prr_block_set *P,
                                   double *scores, prr_block_set *A, prr_block_set *M, float scale,
                                   prr_attn_state *out, void *ws, size_t ws_bytes, const prr_predict_args *pred,
                                   hipStream_t stream) {
    CallTiming timing_;
    if (!q || !meta || !scores || !P || !M) return PRR_EINVAL;
    if (mode != PRR_SCORE_QUEST && mode != PRR_SCORE_MEAN) return PRR_EINVAL;
    PRR_TRY(check_kv(kv));
    PRR_TRY(check_block(kv, block));
    PRR_TRY(check_heads(kv, num_q_heads));
    PRR_TRY(check_set(P));
    PRR_TRY(check_set(A));
    PRR_TRY(check_set(M));
    if (topk < 0 || A->cap < topk || M->cap < topk) return PRR_EINVAL;
    if (!out || !out->acc || !out->l || !out->m) return PRR_EINVAL;
    const int nmax = prr_max_blocks(kv, block);
    if (!selection_plan_exists(kv, nmax, topk, mode == PRR_SCORE_MEAN, true)) return PRR_EUNSUPPORTED;
    if (!ws || ws_bytes < prr_select_spec_workspace_bytes(kv, num_q_heads, block, topk, P->cap))
        return PRR_EWORKSPACE;
    prr::PredictArgs pa;
    PRR_TRY(predict_args(pred, scores, P, A, M, pa));
    PRR_TRY(check_input_set(kv, block, P, stream));
    return hip_status(prr::launch_select_spec(desc(kv), q, num_q_heads, meta, block, prr_meta_stride(kv, block),
                                              nmax, topk, P->idx, P->count, P->pages, P->cap, scores, A->idx,
                                              A->count, A->cap, M->idx, M->count, M->pages, M->cap, scale, out->acc,
                                              out->l, out->m, ws, mode == PRR_SCORE_MEAN, pred ? &pa : nullptr,
                                              stream));
}

size_t prr_layer_step_workspace_bytes(const prr_kv_cache *kv, int32_t num_q_heads, int32_t block, int32_t topk,
                                      int32_t p_cap, int32_t m_cap) {
    if (!kv || kv->batch <= 0 || kv->num_kv_heads <= 0 || num_q_heads <= 0 || kv->head_dim <= 0 ||
        block < prr::kPage || p_cap <= 0 || m_cap <= 0 || topk < 0)
        return 0;
    return prr::layer_step_workspace_bytes(kv->batch, num_q_heads, kv->num_kv_heads, kv->head_dim, block, p_cap, m_cap,
                                           prr_max_blocks(kv, block), topk, kv->dtype == PRR_F32);
}

prr_status prr_layer_step(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, const void *meta,
                          prr_score_mode mode, int32_t block, int32_t topk, const prr_block_set *P, double *scores,
                          prr_block_set *A, prr_block_set *M, float scale, prr_attn_state *state, float *out,
                          void *ws, size_t ws_bytes, const prr_predict_args *pred, hipStream_t stream) {
    CallTiming timing_;
    if (!q || !meta || !scores || !P || !M) return PRR_EINVAL;
    if (mode != PRR_SCORE_QUEST && mode != PRR_SCORE_MEAN) return PRR_EINVAL;
    PRR_TRY(check_kv(kv));
    PRR_TRY(check_block(kv, block));
    PRR_TRY(check_heads(kv, num_q_heads));
    PRR_TRY(check_set(P));
    PRR_TRY(check_set(A));
    PRR_TRY(check_set(M));
    if (topk < 0 || A->cap < topk || M->cap < topk) return PRR_EINVAL;
    if (!state || !state->acc || !state->l || !state->m) return PRR_EINVAL;
    const int nmax = prr_max_blocks(kv, block);
    if (!selection_plan_exists(kv, nmax, topk, mode == PRR_SCORE_MEAN, true)) return PRR_EUNSUPPORTED;
    if (!ws || ws_bytes < prr_layer_step_workspace_bytes(kv, num_q_heads, block, topk, P->cap, M->cap))
        return PRR_EWORKSPACE;
    prr::PredictArgs pa;
    PRR_TRY(predict_args(pred, scores, P, A, M, pa));
    PRR_TRY(check_input_set(kv, block, P, stream));
    return hip_status(prr::launch_layer_step(desc(kv), q, num_q_heads, meta, block, prr_meta_stride(kv, block), nmax,
                                             topk, P->idx, P->count, P->pages, P->cap, scores, A->idx, A->count, A->cap,
                                             M->idx, M->count, M->pages, M->cap, scale, state->acc, state->l,
                                             state->m, out, ws, mode == PRR_SCORE_MEAN, pred ? &pa : nullptr,
                                             stream));
}

prr_status prr_select_spec(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, const void *meta,
                           prr_score_mode mode, int32_t block, int32_t topk, const prr_block_set *P,
                           double *scores, prr_block_set *A, prr_block_set *M, float scale, prr_attn_state *out,
                           void *ws, size_t ws_bytes, hipStream_t stream) {
    CallTiming timing_;
    return prr_select_spec_predict(q, num_q_heads, kv, meta, mode, block, topk, P, scores, A, M, scale, out, ws,
                                   ws_bytes, nullptr, stream);
}

size_t prr_predict_workspace_bytes(int32_t batch, int32_t num_kv_heads, int32_t max_blocks, int32_t budget) {
    if (batch <= 0 || num_kv_heads <= 0 || max_blocks <= 0 || budget < 0) return 0;
    return prr::predict_workspace_bytes(batch, num_kv_heads, max_blocks, budget);
}

prr_status prr_predict(const double *scores, const int32_t *seq_len, int32_t batch,
                       int32_t num_kv_heads, int32_t block, int32_t max_blocks, double alpha,
                       double beta, double gamma, int32_t budget, double *level, double *trend,
                       int32_t *live, prr_block_set *P_next, const prr_kv_cache *kv, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
    CallTiming timing_;
    PRR_TRY(check_predict(scores, seq_len, batch, num_kv_heads, block, max_blocks, budget, level, trend, live,
                          P_next, kv));
    const size_t need = prr::predict_workspace_bytes(batch, num_kv_heads, max_blocks, budget);
    if (ws && ws_bytes < need) return PRR_EWORKSPACE;
    if (max_blocks > prr::kMaxRowTopK && !ws) return PRR_EWORKSPACE;
    const bool listed = P_next->pages != nullptr;
    return hip_status(prr::launch_predict(scores, seq_len, batch, num_kv_heads, block, max_blocks, alpha,
                                          beta, gamma, budget, level, trend, live, P_next->idx,
                                          P_next->count, P_next->pages, P_next->cap,
                                          listed ? kv->page_table : nullptr, listed ? kv->max_pages : 0,
                                          need ? ws : nullptr, stream));
}

prr_status prr_spec_attn(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, int32_t block,
                         const prr_block_set *P, float scale, prr_attn_state *out, void *ws,
                         size_t ws_bytes, hipStream_t stream) {
    CallTiming timing_;
    PRR_TRY(attn_common(q, num_q_heads, kv, block, P, ws, ws_bytes));
    if (!out || !out->acc || !out->l || !out->m) return PRR_EINVAL;
    PRR_TRY(check_input_set(kv, block, P, stream));
    return hip_status(prr::launch_attn(desc(kv), q, num_q_heads, block, P->idx, P->count, P->pages, P->cap, scale,
                                       out->acc, out->l, out->m, nullptr, false, ws, stream));
}

prr_status prr_spec_attn_noalloc(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, int32_t block,
                                 const prr_block_set *P, float scale, prr_attn_state *out, hipStream_t stream) {
    CallTiming timing_;
    static_assert(PRR_NOALLOC_SCRATCH_BYTES == prr::kNoAllocScratchBytes, "scratch size");
    if (!q) return PRR_EINVAL;
    PRR_TRY(check_kv(kv));
    PRR_TRY(check_block(kv, block));
    PRR_TRY(check_heads(kv, num_q_heads));
    PRR_TRY(check_set(P));
    if (!out || !out->acc || !out->l || !out->m) return PRR_EINVAL;
    if (prr::attn_workspace_bytes(kv->batch, num_q_heads, kv->num_kv_heads, kv->head_dim, block, P->cap) >
        prr::kNoAllocScratchBytes)
        return PRR_EWORKSPACE;
    PRR_TRY(check_input_set(kv, block, P, stream));
    return hip_status(prr::launch_spec_noalloc(desc(kv), q, num_q_heads, block, P->idx, P->count, P->pages, P->cap,
                                               scale, out->acc, out->l, out->m, stream));
}

prr_status prr_repair(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, int32_t block,
                      const prr_block_set *M, float scale, prr_attn_state *state, float *out,
                      void *ws, size_t ws_bytes, hipStream_t stream) {
    CallTiming timing_;
    PRR_TRY(attn_common(q, num_q_heads, kv, block, M, ws, ws_bytes));
    if (!state || !state->acc || !state->l || !state->m) return PRR_EINVAL;
    PRR_TRY(check_input_set(kv, block, M, stream));
    return hip_status(prr::launch_attn(desc(kv), q, num_q_heads, block, M->idx, M->count, M->pages, M->cap, scale,
                                       state->acc, state->l, state->m, out, true, ws, stream));
}

size_t prr_calibrate_workspace_bytes(int32_t rows, int32_t blocks, int32_t n_candidates) {
    if (rows <= 0 || blocks <= 0 || n_candidates <= 0) return 0;
    return prr::calib_workspace_bytes(rows, blocks, n_candidates);
}

prr_status prr_calibrate(const float *scores, int32_t rows, int32_t blocks, int32_t topk, const double *grid,
                         int32_t n_candidates, double *H, int32_t *best, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
    CallTiming timing_;
    if (!scores || !grid || !H || !best) return PRR_EINVAL;
    if (rows <= 0 || blocks <= 0 || topk < 0 || n_candidates <= 0) return PRR_EINVAL;
    if (blocks > prr::kMaxCalibBlocks || n_candidates > prr::kMaxCalibGrid) return PRR_EUNSUPPORTED;
    if ((int64_t)rows * blocks > INT32_MAX) return PRR_EUNSUPPORTED;
    if (!ws || ws_bytes < prr::calib_workspace_bytes(rows, blocks, n_candidates)) return PRR_EWORKSPACE;
    return hip_status(prr::launch_calibrate(scores, rows, blocks, topk, grid, n_candidates, H, best, ws, stream));
}

const char *prr_strerror(prr_status status) {
    switch (status) {
        case PRR_OK: return "ok";
        case PRR_EINVAL: return "invalid argument";
        case PRR_EUNSUPPORTED: return "unsupported shape or dtype";
        case PRR_EWORKSPACE: return "workspace missing or too small";
        case PRR_EHIP: return "HIP launch or runtime error";
    }
    return "unknown status";
}

}  // extern "C"
