// step_layer.hip - the layer step as one launch for bf16 caches (gfx950): selection, the speculative pass over
// P and repair over M = A \ P in one grid.  The device code and its design notes are in step_core.hpp and
// attn_core.hpp; fp8 caches are instantiated in step_layer_fp8.hip, and an fp32 cache runs the calls in turn.

#include "step_core.hpp"

namespace prr {

size_t layer_step_workspace_bytes(int batch, int hq, int hkv, int d, int block, int p_cap, int m_cap, int nmax,
                                  int topk, bool f32) {
    const size_t units = (size_t)batch * hkv;
    return select_spec_workspace_bytes(batch, hq, hkv, d, block, p_cap, nmax, topk, f32) +
           layer_extra_m_ws(batch, hq, hkv, d, block, m_cap) + units * 4 * kReadyStride + 256;
}

hipError_t launch_layer_step(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride, int nmax,
                             int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap, double *scores,
                             int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx, int32_t *m_cnt, int32_t *m_pages, int m_cap,
                             float scale, float *acc, float *l, float *m, float *out, void *ws, bool mean,
                             const PredictArgs *pred, hipStream_t stream) {
    void *mws = (char *)ws + select_spec_workspace_bytes(kv.batch, hq, kv.hkv, kv.d, block, p_cap, nmax, topk,
                                                         !kv.bf16 && !kv.fp8);
    if (kv.fp8)
        return launch_layer_step_fp8(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores, a_idx,
                                     a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, out, ws, mws, mean, pred,
                                     stream);
    if (kv.bf16)
        return launch_layer_step_t<kKtBf16>(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores,
                                            a_idx, a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, out, ws, mws,
                                            mean, pred, stream);
    // fp32 caches (exact-input checks): prr_select_spec's passes, then prr_repair's
    hipError_t e = launch_select_spec(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores, a_idx,
                                      a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, ws, mean, pred, stream);
    if (e != hipSuccess) return e;
    return launch_attn(kv, q, hq, block, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, out, true, mws, stream);
}

}  // namespace prr
