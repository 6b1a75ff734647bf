// Internal launch interface between the C ABI (prr_api.cpp) and the kernels.  Host-side only types.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace prr {

// Kernel timing (prr_time_next_kernel): the start event goes to the first kernel an entry-point call
// launches, the stop event to every kernel it launches (the last one's end remains).  false when none
// are armed for the calling thread's current call.
bool take_kernel_timing(hipEvent_t *start, hipEvent_t *stop);

template <typename T>
struct same_type {
    typedef T type;
};

// Launches `kernel` on `stream`; when timing events are armed for the current entry-point call, through
// hipExtLaunchKernel with them, so that they hold kernel start and end times.  The arguments
// are converted to the kernel's parameter types at the call.
template <typename... Params>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream,
                  typename same_type<Params>::type... args) {
    hipEvent_t start = nullptr, stop = nullptr;
    if (take_kernel_timing(&start, &stop)) {
        void *argv[] = {(void *)&args..., nullptr};
        hipError_t e = hipExtLaunchKernel((const void *)kernel, grid, block, argv, 0, stream, start, stop, 0);
        if (e != hipSuccess) return e;
    } else {
        kernel<<<grid, block, 0, stream>>>(args...);
    }
    return hipGetLastError();
}

// launch(...) inside a function returning hipError_t: returns the launch's error, if any.
#define PRR_LAUNCH(...)                                     \
    do {                                                    \
        const hipError_t prr_e_ = ::prr::launch(__VA_ARGS__); \
        if (prr_e_ != hipSuccess) return prr_e_;           \
    } while (0)

// Compute units of the current device (the launch shapes spread work over them), queried once per
// device and kept: a device property, not state that calls change.
int device_cu_count();

constexpr int kPage = 16;          // tokens per page (the only supported page size)
constexpr int kMaxRowTopK = 32768; // blocks per (sequence, kv head) one top-K workgroup holds on chip
constexpr int kMaxSelectN = 131072; // blocks per (sequence, kv head) selection and the predictor take;
                                    // rows longer than kMaxRowTopK are ranked in part-parallel stages
constexpr int kStagedSelectMin = 8192; // prr_select ranks rows longer than this in stages when given a
                                       // workspace (one top-K workgroup per unit leaves most CUs idle)
constexpr int kMaxCalibBlocks = 4096; // calibration: blocks per prefill row (16 per thread of four waves)
constexpr int kMaxCalibGrid = 4096;   // calibration: candidates (alpha, beta, gamma)

struct KvDesc {
    const void *k;
    const void *v;
    const int32_t *page_table;
    const int32_t *seq_len;
    int batch, hkv, d, num_pages, max_pages;
    bool bf16;   // bf16 K/V and queries
    bool fp8;    // E4M3 K/V, bf16 queries and metadata
};

// Attention workspace: 2 x [units] uint32 counters (chunk arrivals, scoring arrivals), padded to 256 B,
// then one partial state per chunk.
size_t attn_workspace_bytes(int batch, int hq, int hkv, int d, int block, int cap);

// pages (may be null): the set's page work list.
hipError_t launch_attn(const KvDesc &kv, const void *q, int hq, int block, const int32_t *idx,
                       const int32_t *count, const int32_t *pages, int cap, float scale, float *acc, float *l,
                       float *m, float *out, bool repair, void *ws, hipStream_t stream);

hipError_t launch_clear(void *ws, size_t bytes, hipStream_t stream);

// The speculative pass with the library's own per-device buffer of kNoAllocScratchBytes as its workspace
// (prr_spec_attn_noalloc); the caller has checked that attn_workspace_bytes fits.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t launch_spec_noalloc(const KvDesc &kv, const void *q, int hq, int block, const int32_t *idx,
                               const int32_t *count, const int32_t *pages, int cap, float scale, float *acc,
                               float *l, float *m, hipStream_t stream);

// Checking mode (PRR_CHECK=1 in the environment): validates a block set on the stream and waits for the
// result; *violation gets a bit mask (1 count outside [0, cap], 2 entry out of range, 4 repeated entry).
bool checks_enabled();
hipError_t check_sets(const KvDesc &kv, int block, const int32_t *idx, const int32_t *count, int cap,
                      hipStream_t stream, int *violation);

// Block metadata: min/max keys ([d][2][stride] per unit, cache dtype) or, mean = true, the fp32 block
// means ([d][stride] per unit).
hipError_t launch_meta(const KvDesc &kv, int block, int stride, void *meta, bool mean, hipStream_t stream);

// Scoring and top-K (prr_select).  Without ws (rows of up to kMaxRowTopK blocks): the score kernel, then
// one top-K workgroup per unit.  With ws (select_workspace_bytes of caller memory, zeroed once; every call
// leaves it so), rows longer than kStagedSelectMin: every scoring workgroup keeps its part's local top-K
// candidates, then groups of parts and the unit's final ranking (three stages, as a fused launch's).
hipError_t launch_select(const KvDesc &kv, const void *q, int hq, const void *meta, int block,
                         int stride, int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt,
                         int p_cap, double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap,
                         int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap, bool mean, void *ws,
                         hipStream_t stream);

// Top-K + M = A \ P from scores already in place (the second half of launch_select).  m_pages (may be
// null): M's page work list, written with M.
hipError_t launch_topk(const KvDesc &kv, int block, int nmax, int topk, const double *scores,
                       const int32_t *p_idx, const int32_t *p_cnt, int p_cap, int32_t *a_idx, int32_t *a_cnt,
                       int a_cap, int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap, hipStream_t stream);

// How prr_select_spec ranks a unit's blocks: kpt keys per thread inside the launch (two: over candidates
// of a two-stage top-K with kl candidates per scoring workgroup), or kpt = 0: the separate top-K kernel.
struct SelectSpecPlan {
    bool two;
    int kl;
    int kpt;
    // three stages (rows with more candidate slots than one ranking holds): the launch keeps the parts'
    // candidates only (kpt = 0); then ng groups of gp parts per unit keep their top-kl2 each (kpt2 slots per
    // thread) and the unit's last group ranks the ng kl2 group candidates (kpt3 slots per thread).
    bool three;
    int gp, ng, kl2, kpt2, kpt3;
    int bpw;   // blocks per scoring workgroup (score_bpw: 1024 for wide bf16 min/max scoring)
};
SelectSpecPlan select_spec_plan(int nmax, int topk, bool mean, int units);

// The staged plan of launch_select for rows of more than kStagedSelectMin blocks (three stages; wide
// scoring parts for bf16 min/max rows of kWideScoreBlocks and more where they have a plan).
SelectSpecPlan select_stage_plan(int nmax, int topk, bool bq, bool mean);

// The plan for parts of bpw blocks.  force_three: the three stages even where two would do, for a top-K
// that ranks in launches of its own (rows longer than kMaxTwoStageBlocks, whose P bitmap only those
// launches hold).  No plan (two false): more candidates than the stages rank.
SelectSpecPlan stage_plan(int nmax, int topk, int bpw, bool force_three);

// Where a three-stage top-K keeps its data, from base: the parts' candidates (nparts per unit; keys,
// then indices, then counts), the groups' (same layout), one group arrival counter per unit, then (for a
// fused launch that runs the stages itself) one part arrival counter per group, each 256-byte aligned.
// bytes: the whole.
struct StageLayout {
    char *cand1, *cand2;
    uint32_t *garr, *parr;
    size_t bytes;
};
inline StageLayout stage_layout(char *base, int units, int nparts, const SelectSpecPlan &pl) {
    const auto align = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t parts = (size_t)units * nparts, groups = (size_t)units * pl.ng;
    const size_t b1 = align(parts * pl.kl * 12 + parts * 4);
    const size_t b2 = align(groups * pl.kl2 * 12 + groups * 4);
    const size_t b3 = align((size_t)units * 4);
    StageLayout l;
    l.cand1 = base;
    l.cand2 = base + b1;
    l.garr = (uint32_t *)(base + b1 + b2);
    l.parr = (uint32_t *)(base + b1 + b2 + b3);
    l.bytes = b1 + b2 + b3 + align(groups * 4);
    return l;
}

// launch_select's workspace: 0 for rows of up to kStagedSelectMin blocks and where the stages have no
// plan, else the three stages' (stage_layout over parts of the score kernel's size).  bq: bf16 queries
// and metadata.  select_supported: whether launch_select has a plan for the shape.
size_t select_workspace_bytes(int units, int nmax, int topk, bool bq, bool mean);
bool select_supported(int nmax, int topk, bool bq, bool mean);

// The second and third stages of a three-stage top-K (plan.three): nparts parts of kl candidates per
// unit at cand1 (keys, then indices, then counts, as the fused launch writes them); the group candidates
// go to cand2 (same layout, ng x kl2 slots per unit), the per-unit group arrival counters to arrivals
// (zero at rest; the last group of a unit resets its counter).  live (a predictor step's, may be null):
// set to the unit's block count by its last group.
hipError_t launch_topk_groups(const KvDesc &kv, int block, int nmax, int topk, const int32_t *p_idx,
                              const int32_t *p_cnt, int p_cap, int32_t *a_idx, int32_t *a_cnt, int32_t *a_pages,
                              int a_cap, int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap,
                              const SelectSpecPlan &plan, int nparts,
                              void *cand1, void *cand2, uint32_t *arrivals, hipStream_t stream,
                              int32_t *live = nullptr);

// Offset of the carried predictor's work counter in the prr_select_spec workspace.
size_t pred_counter_offset(int batch, int hq, int hkv, int d, int block, int cap, int nmax, int topk, bool f32);

// Workspace of prr_select_spec: the speculative pass's attention workspace, then (two-stage top-K) the
// candidates of every scoring workgroup, or for an fp32 cache (f32) launch_select's workspace.
size_t select_spec_workspace_bytes(int batch, int hq, int hkv, int d, int block, int cap, int nmax, int topk,
                                   bool f32);

// Selection and the speculative pass over P in one grid (bf16 caches; fp32 caches run the two in turn),
// then the top-K.  ws: select_spec_workspace_bytes.
// One predictor step (the arguments of launch_predict), for a launch that carries it along.
struct PredictArgs {
    const double *scores;
    const int32_t *seq_len;
    int batch, hkv, block, nmax, budget;
    double alpha, beta, gamma;
    double *level;
    double *trend;
    int32_t *live;
    int32_t *p_idx;
    int32_t *p_cnt;
    int p_cap;
    void *ws;   // predictor workspace for long rows (may be null)
    int32_t *p_pages;             // P's page work list (may be null), through page_table [batch][max_pages]
    const int32_t *page_table;
    int max_pages;
};

// Rows of at most this many blocks let the predictor step run inside the selection + speculative launch.
constexpr int kMaxFusedPredictN = 2048;

// pred (may be null): a predictor step over other buffers, run by extra workgroups of the same launch
// when its rows fit (kMaxFusedPredictN), else as its own launch after it on the stream.
hipError_t launch_select_spec(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride,
                              int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap,
                              double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx,
                              int32_t *m_cnt, int32_t *m_pages, int m_cap, float scale, float *acc, float *l, float *m,
                              void *ws, bool mean, const PredictArgs *pred, hipStream_t stream);

// The fused launch for fp8 caches (compiled in its own file; arguments as launch_select_spec).
hipError_t launch_select_spec_fp8(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride,
                                  int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap,
                                  double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx,
                                  int32_t *m_cnt, int32_t *m_pages, int m_cap, float scale, float *acc, float *l, float *m, void *ws,
                                  bool mean, const PredictArgs *pred, hipStream_t stream);

// The layer step (selection, the speculative pass over P, repair over M) in one launch where the top-K
// finishes inside it (bf16 and fp8 caches), else as the select_spec launches followed by repair's.  The
// final state over P u M goes to acc, l, m, the normalised output to out (may be null).  ws:
// layer_step_workspace_bytes: the select_spec workspace, then M's attention workspace, the per-unit M flags
// and a status word (zeroed once; every call leaves it ready for the next).
size_t layer_step_workspace_bytes(int batch, int hq, int hkv, int d, int block, int p_cap, int m_cap, int nmax,
                                  int topk, bool f32);
hipError_t launch_layer_step(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride, int nmax,
                             int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap, double *scores,
                             int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap,
                             float scale, float *acc, float *l, float *m, float *out, void *ws, bool mean,
                             const PredictArgs *pred, hipStream_t stream);
// fp8 caches (compiled in its own file); mws: the M part of the workspace
hipError_t launch_layer_step_fp8(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride,
                                 int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap,
                                 double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx,
                                 int32_t *m_cnt, int32_t *m_pages, int m_cap, float scale, float *acc, float *l, float *m, float *out,
                                 void *ws, void *mws, bool mean, const PredictArgs *pred, hipStream_t stream);

// ws (may be null): rows longer than 2048 blocks are then updated by 512-block parts in parallel and
// ranked in two stages (predict_workspace_bytes; 0 where one workgroup per unit is used regardless).
size_t predict_workspace_bytes(int batch, int hkv, int nmax, int budget);
// p_pages (may be null): P's page work list, written with P through page_table ([batch][max_pages]).
hipError_t launch_predict(const double *scores, const int32_t *seq_len, int batch, int hkv,
                          int block, int nmax, double alpha, double beta, double gamma, int budget,
                          double *level, double *trend, int32_t *live, int32_t *p_idx,
                          int32_t *p_cnt, int32_t *p_pages, int p_cap, const int32_t *page_table, int max_pages,
                          void *ws, hipStream_t stream);

// Decode append: token seq_len[b] of every sequence into the cache and its block's metadata, then
// seq_len[b] += 1.
hipError_t launch_append(const KvDesc &kv, void *k, void *v, int32_t *seq_len, const void *k_new,
                         const void *v_new, int block, int stride, void *meta, bool mean, hipStream_t stream);

// Calibration workspace: A-set masks per row, EMA checkpoints per (candidate, chunk), chunk sums.
size_t calib_workspace_bytes(int rows, int blocks, int n);

hipError_t launch_calibrate(const float *scores, int rows, int blocks, int k, const double *grid, int n,
                            double *H, int32_t *best, void *ws, hipStream_t stream);

}  // namespace prr
