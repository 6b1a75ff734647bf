// step_layer_fp8.hip - the layer step as one launch for fp8 (E4M3) caches (gfx950): the device code of
// step_core.hpp instantiated for fp8 tiles, compiled apart from the bf16 variants.

#include "step_core.hpp"

namespace prr {

hipError_t launch_layer_step_fp8(const KvDesc &kv, const void *q, int hq, const void *meta, int block, int stride,
                                 int nmax, int topk, const int32_t *p_idx, const int32_t *p_cnt, const int32_t *p_pages, int p_cap,
                                 double *scores, int32_t *a_idx, int32_t *a_cnt, int a_cap, int32_t *m_idx,
                                 int32_t *m_cnt, int32_t *m_pages, int m_cap, float scale, float *acc, float *l, float *m, float *out,
                                 void *ws, void *mws, bool mean, const PredictArgs *pred, hipStream_t stream) {
    return launch_layer_step_t<kKtFp8>(kv, q, hq, meta, block, stride, nmax, topk, p_idx, p_cnt, p_pages, p_cap, scores, a_idx,
                                       a_cnt, a_cap, m_idx, m_cnt, m_pages, m_cap, scale, acc, l, m, out, ws, mws, mean, pred,
                                       stream);
}

}  // namespace prr
