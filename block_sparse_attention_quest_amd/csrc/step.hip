// step.hip - selection and the speculative pass over P as one launch (gfx950).
//
// Citations:
//   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
//           Decoding" (full paper text)
//
// The method overlaps the speculative pass over the predicted set P with selection ([paper] §1 and the
// Figure 1 flow, §3): the two only read P and are independent.  On this GPU a dependency between two
// streams costs about 10 us from the producer's end to the consumer's start, while kernels on one
// stream follow each other about 1 us apart, so the overlap is made inside one grid instead: the first
// workgroups run the speculative chunks (the attention kernels' chunk walk over n_spec workgroups),
// the rest score blocks (one workgroup per 256 blocks of a unit).  Dispatch follows the workgroup
// index, so the speculative workgroups are resident first, about one per CU, and the scoring
// workgroups stream through the remaining slots.  Both parts are HBM-bound; their prologues and tails
// overlap each other's streaming.  The top-K (with M = A \ P) follows as its own kernel on the same
// stream.

#include "select_core.hpp"
#include "attn_core.hpp"

namespace prr {
namespace {

// Workgroups [0, n_spec) run the speculative pass; workgroup n_spec + s scores blocks
// [256 (s mod nsx), +256) of unit s / nsx.  Register use is the attention part's (two waves per SIMD).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void select_spec_kernel(
    AttnParams ap, ScoreParams sp, int n_spec, int nsx) {
    if ((int)blockIdx.x < n_spec) {
        attn_body<true, D, false>(ap, blockIdx.x, n_spec);
        return;
    }
    const int s = (int)blockIdx.x - n_spec;
    score_body<true, D>(sp, s % nsx, s / nsx);
}

}  // namespace

hipError_t launch_select_spec(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride,
                              int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt, int p_cap,
                              double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx,
                              int32_t *m_cnt, int m_cap, float scale, float *acc, float *l, float *m,
                              void *ws, hipStream_t stream) {
    if (!kv.bf16) {
        // fp32 caches (exact-input checks): the two passes one after the other
        hipError_t e = launch_select(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_cap, scores,
                                     a_idx, a_cnt, a_cap, m_idx, m_cnt, m_cap, stream);
        if (e != hipSuccess) return e;
        return launch_attn(kv, q, hq, block, p_idx, p_cnt, p_cap, scale, acc, l, m, nullptr, false, ws, stream);
    }
    AttnParams ap;
    const int n_spec = attn_setup(ap, kv, q, hq, block, p_idx, p_cnt, p_cap, scale, acc, l, m, nullptr, false, ws);
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
    const int units = kv.batch * kv.hkv;
    const int nsx = (nmax + 255) / 256;
    const long grid = (long)n_spec + (long)nsx * units;
    if (grid > 0x7fffffffL) return hipErrorInvalidValue;
    if (kv.d == 128) select_spec_kernel<128><<<(int)grid, 256, 0, stream>>>(ap, sp, n_spec, nsx);
    else select_spec_kernel<64><<<(int)grid, 256, 0, stream>>>(ap, sp, n_spec, nsx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk(kv, block, nmax, topk, scores, p_idx, p_cnt, p_cap, a_idx, a_cnt, a_cap, m_idx, m_cnt,
                       m_cap, stream);
}

}  // namespace prr
