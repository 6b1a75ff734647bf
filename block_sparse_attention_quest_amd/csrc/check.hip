// check.hip - checking mode for the device-side preconditions of block sets (gfx950).
//
// Block sets come from the caller or from other entry points; their entries are indices of blocks that
// exist.  The kernels do not verify that (an entry out of range or repeated is the caller's contract).
// With PRR_CHECK=1 in the environment the entry points first run check_sets_kernel on every input set
// and return PRR_EINVAL, before the real work is enqueued, if a set's count lies outside [0, cap], an
// entry lies outside [0, ceil(seq_len / block)), or an entry repeats.  The mode waits for the check's
// result on the stream, so it is meant for debugging, not for the decode loop.  Calls in checking mode
// share one result word and must not overlap.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "prr_internal.hpp"

namespace prr {
namespace {

__device__ int g_set_violation;   // bit 0: count, bit 1: range, bit 2: repeat

// One workgroup per (sequence, kv head) unit; repeats by pairwise comparison (sets hold at most a few
// thousand entries), reads clamped to the set's capacity.
__global__ __launch_bounds__(256) void check_sets_kernel(const int32_t *idx, const int32_t *count, int cap,
                                                         const int32_t *seq_len, int hkv, int block) {
    const int u = blockIdx.x;
    const int b = u / hkv;
    const int cnt_raw = count[u];
    int bad = 0;
    if (cnt_raw < 0 || cnt_raw > cap) bad |= 1;
    const int cnt = min(max(cnt_raw, 0), cap);
    const long nb = ((long)max(seq_len[b], 0) + block - 1) / block;
    const int32_t *row = idx + (size_t)u * cap;
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
        const int32_t x = row[i];
        if (x < 0 || (long)x >= nb) bad |= 2;
        for (int j = 0; j < i; ++j)
            if (row[j] == x) {
                bad |= 4;
                break;
            }
    }
    if (bad) atomicOr(&g_set_violation, bad);
}

__global__ void clear_violation_kernel() { g_set_violation = 0; }

}  // namespace

bool checks_enabled() {
    static const bool on = [] {
        const char *v = getenv("PRR_CHECK");
        return v && atoi(v) == 1;
    }();
    return on;
}

hipError_t check_sets(const KvDesc &kv, int block, const int32_t *idx, const int32_t *count, int cap,
                      hipStream_t stream, int *violation) {
    *violation = 0;
    const int units = kv.batch * kv.hkv;
    clear_violation_kernel<<<1, 1, 0, stream>>>();
    check_sets_kernel<<<units, 256, 0, stream>>>(idx, count, cap, kv.seq_len, kv.hkv, block);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipMemcpyFromSymbolAsync(violation, HIP_SYMBOL(g_set_violation), sizeof(int), 0, hipMemcpyDeviceToHost,
                                 stream);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(stream);
}

}  // namespace prr
