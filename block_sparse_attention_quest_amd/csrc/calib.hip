// calib.hip - online predictor calibration on the GPU (gfx950).  Compiled with -ffp-contract=off:
// every float64 multiply and add is separately rounded, in the order the comments state, so the EMA
// trajectories (and therefore every predicted set) are bit-identical to a plain float64 evaluation.
//
// Citations:
//   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
//           Decoding" (full paper text), §4.2 online predictor calibration
//   [blog]  "PRR: Predict, Reuse, and Repair - Accelerating Dynamic Sparse Attention for Long-Context
//           LLM Decoding" (xllm-io paper review), Eqs. (4)-(5)
//
// What is computed.  The prefill score matrix IS[rows][blocks] is a trajectory of block scores.  For
// each candidate theta = (alpha, beta, gamma) of a grid, an EMA level/trend predictor runs over the
// rows: row 0 sets level = IS_0, trend = 0; every later row phi is first predicted
// (level + gamma trend, [paper] §4.1), the predicted top-K set P_phi is compared with the true top-K
// set A_phi of the row by the score-weighted hit rate h_phi = sum_{b in P n A} IS / sum_{b in A} IS
// ([paper] §4.2, [blog] Eq. (4)), and the row is then absorbed with the level/trend update.  H(theta)
// is the mean of h over rows 1 .. rows-1 and theta* the first argmax in grid order ([blog] Eq. (5)).
//
// How it maps to the GPU.  The EMA of one (theta, block) is a sequential scalar recurrence, but the
// top-K sets of different rows are independent.  Four launches:
//   1. rows_topk:  one wave per row, A_phi as a bit mask (a wave-level radix select);
//   2. ema_chain:  one thread per (theta, block) runs the recurrence over all rows and stores the state
//                  at the start of every chunk of kChunk rows (checkpoints);
//   3. replay:     one wave per (theta, chunk) resumes from its checkpoint with the same operations,
//                  predicts, selects P_phi (wave radix select), and sums h over its rows;
//   4. finish:     H = sum of the chunk sums / (rows - 1) per theta, and the first argmax.
// Top-K ties go to the smaller block index; hit-rate sums use the same reduction tree for numerator
// and denominator, so P = A gives h = 1 exactly.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "prr_internal.hpp"

#pragma clang fp contract(off)

namespace prr {
namespace {

constexpr int kCalibChunk = 64;   // rows per replay wave

__device__ __forceinline__ double dadd(double a, double b) {
#pragma clang fp contract(off)
    return a + b;
}
__device__ __forceinline__ double dmul(double a, double b) {
#pragma clang fp contract(off)
    return a * b;
}
__device__ __forceinline__ double dsub(double a, double b) {
#pragma clang fp contract(off)
    return a - b;
}

// Order-preserving image of a double (larger double -> larger key); -0.0 maps with +0.0.
__device__ __forceinline__ uint64_t order_key(double x) {
    uint64_t b = (uint64_t)__double_as_longlong(x);
    if (b == 0x8000000000000000ull) b = 0;
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int o) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = dadd(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint64_t spread16(uint32_t x) {
    return (uint64_t)(x & 0xffu) | ((uint64_t)(x & 0xff00u) << 8) | ((uint64_t)(x & 0xff0000u) << 16) |
           ((uint64_t)(x & 0xff000000u) << 24);
}

// The k largest of n keys held by one wave (key descending, index ascending); lane l holds indices
// [l KPL, l KPL + KPL).  MSD radix select with 4-bit digits over the bits where the keys differ;
// per-lane digit counts are packed 8-bit fields, widened to 16 bits for the cross-lane sums.  Returns
// the lane's KPL-bit selection mask.
template <int KPL>
__device__ uint32_t wave_topk(const uint64_t (&key)[KPL], int n, int k) {
    const int lane = threadIdx.x & 63;
    const int base = lane * KPL;
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
        if (base + j < n) valid |= 1u << j;
    if (k <= 0) return 0u;
    if (k >= n) return valid;

    uint64_t a = ~0ull, o = 0ull;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
        if (valid >> j & 1u) {
            a &= key[j];
            o |= key[j];
        }
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) {
        a &= shfl_xor64(a, s);
        o |= shfl_xor64(o, s);
    }
    const uint64_t diff = a ^ o;
    uint64_t prefix, mask;
    int remaining = k;
    bool take_all = false;
    if (diff == 0) {
        prefix = a;
        mask = ~0ull;
    } else {
        const int top = 63 - __clzll((long long)diff);
        int shift = (top / 4) * 4;
        mask = shift + 4 >= 64 ? 0ull : ~((1ull << (shift + 4)) - 1ull);
        prefix = a & mask;
        for (; shift >= 0; shift -= 4) {
            uint64_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                if ((valid >> j & 1u) && (key[j] & mask) == prefix) {
                    const uint32_t d = (uint32_t)(key[j] >> shift) & 15u;
                    const uint64_t inc = 1ull << ((d & 7u) * 8u);
                    if (d & 8u) hi += inc;
                    else lo += inc;
                }
            }
            const uint64_t w0 = spread16((uint32_t)lo), w1 = spread16((uint32_t)(lo >> 32));
            const uint64_t w2 = spread16((uint32_t)hi), w3 = spread16((uint32_t)(hi >> 32));
            uint32_t c8[8] = {(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32),
                              (uint32_t)w2, (uint32_t)(w2 >> 32), (uint32_t)w3, (uint32_t)(w3 >> 32)};
#pragma unroll
            for (int i = 0; i < 8; ++i) c8[i] = wave_sum_u32(c8[i]);
            uint32_t cnt[16];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                cnt[2 * i] = c8[i] & 0xffffu;
                cnt[2 * i + 1] = c8[i] >> 16;
            }
            int dsel = 0;
            uint32_t cum = 0, csel = 0;
            bool found = false;
#pragma unroll
            for (int d = 15; d >= 0; --d) {
                if (!found) {
                    if (cum + cnt[d] >= (uint32_t)remaining) {
                        dsel = d;
                        csel = cnt[d];
                        found = true;
                    } else {
                        cum += cnt[d];
                    }
                }
            }
            remaining -= (int)cum;
            prefix |= (uint64_t)dsel << shift;
            mask |= 15ull << shift;
            if (csel == (uint32_t)remaining) {
                take_all = true;
                break;
            }
        }
    }
    uint32_t sel = 0, tie = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        if (!(valid >> j & 1u)) continue;
        const uint64_t mk = key[j] & mask;
        if (mk > prefix) sel |= 1u << j;
        else if (mk == prefix) tie |= 1u << j;
    }
    if (take_all) return sel | tie;
    // ties on the full key: the `remaining` smallest indices win (exclusive scan over lanes)
    const uint32_t my = __popc(tie);
    uint32_t incl = my;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const uint32_t y = __shfl_up(incl, s);
        if (lane >= s) incl += y;
    }
    uint32_t r = incl - my;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
        if (tie >> j & 1u) {
            if (r < (uint32_t)remaining) sel |= 1u << j;
            ++r;
        }
    return sel;
}

struct CalibParams {
    const float *scores;    // [rows][blocks]
    const double *grid;     // [n][3]: alpha, beta, gamma
    double *H;              // [n]
    int32_t *best;          // [1]
    uint32_t *amask;        // [rows][64]: lane l's KPL-bit share of A_phi
    double *ckpt;           // [n][nchunks][2][blocks]: level, trend at the start of each chunk
    double *partial;        // [n][nchunks]
    int rows, blocks, k, n, nchunks;
};

// 1. A_phi = top-k of row phi (phi >= 1), one wave per row.
template <int KPL>
__global__ __launch_bounds__(256) void rows_topk_kernel(CalibParams p) {
    const int lane = threadIdx.x & 63;
    const int phi = 1 + blockIdx.x * 4 + (threadIdx.x >> 6);
    if (phi >= p.rows) return;
    const float *row = p.scores + (size_t)phi * p.blocks;
    uint64_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int b = lane * KPL + j;
        key[j] = b < p.blocks ? order_key((double)row[b]) : 0ull;
    }
    p.amask[(size_t)phi * 64 + lane] = wave_topk<KPL>(key, p.blocks, p.k);
}

// 2. The EMA recurrence of one (theta, block) over all rows, with a checkpoint at every chunk start.
// Chunk c covers rows [1 + c kCalibChunk, 1 + (c + 1) kCalibChunk); its checkpoint is the state after
// absorbing rows 0 .. c kCalibChunk.
__global__ __launch_bounds__(256) void ema_chain_kernel(CalibParams p) {
    const int gid = blockIdx.x * 256 + threadIdx.x;
    if (gid >= p.n * p.blocks) return;
    const int th = gid / p.blocks, b = gid - th * p.blocks;
    const double alpha = p.grid[3 * th], beta = p.grid[3 * th + 1];
    const double one_a = dsub(1.0, alpha), one_b = dsub(1.0, beta);
    double level = (double)p.scores[b];   // row 0: level = IS_0, trend = 0
    double trend = 0.0;
    double *ck = p.ckpt + (size_t)th * p.nchunks * 2 * p.blocks + b;
    ck[0] = level;
    ck[p.blocks] = trend;
    for (int phi = 1; phi < p.rows; ++phi) {
        const double is = (double)p.scores[(size_t)phi * p.blocks + b];
        // trend = beta (IS - level_old) + (1 - beta) trend;  level = alpha IS + (1 - alpha) level_old
        const double t = dsub(is, level);
        trend = dadd(dmul(beta, t), dmul(one_b, trend));
        level = dadd(dmul(alpha, is), dmul(one_a, level));
        if (phi % kCalibChunk == 0) {
            const int c = phi / kCalibChunk;
            if (c < p.nchunks) {
                ck[(size_t)c * 2 * p.blocks] = level;
                ck[(size_t)c * 2 * p.blocks + p.blocks] = trend;
            }
        }
    }
}

// 3. One wave per (theta, chunk): predict, select P_phi, score-weighted hit rate, absorb the row.
template <int KPL>
__global__ __launch_bounds__(256) void replay_kernel(CalibParams p) {
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= p.n * p.nchunks) return;
    const int th = item / p.nchunks, c = item - th * p.nchunks;
    const double alpha = p.grid[3 * th], beta = p.grid[3 * th + 1], gamma = p.grid[3 * th + 2];
    const double one_a = dsub(1.0, alpha), one_b = dsub(1.0, beta);
    const double *ck = p.ckpt + ((size_t)th * p.nchunks + c) * 2 * p.blocks;
    double level[KPL], trend[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int b = min(lane * KPL + j, p.blocks - 1);
        level[j] = ck[b];
        trend[j] = ck[p.blocks + b];
    }
    const int phi0 = 1 + c * kCalibChunk;
    const int phi1 = min(p.rows, phi0 + kCalibChunk);
    double sum = 0.0;
    for (int phi = phi0; phi < phi1; ++phi) {
        uint64_t key[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) key[j] = order_key(dadd(level[j], dmul(gamma, trend[j])));   // prediction
        const uint32_t pm = wave_topk<KPL>(key, p.blocks, p.k);
        const uint32_t am = p.amask[(size_t)phi * 64 + lane];
        const float *row = p.scores + (size_t)phi * p.blocks;
        double is[KPL];
        double num = 0.0, den = 0.0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const int b = lane * KPL + j;
            is[j] = b < p.blocks ? (double)row[b] : 0.0;
            if (am >> j & 1u) {
                den = dadd(den, is[j]);
                num = dadd(num, (pm >> j & 1u) ? is[j] : 0.0);
            }
        }
        num = wave_sum_f64(num);
        den = wave_sum_f64(den);
        sum = dadd(sum, den != 0.0 ? num / den : 0.0);
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const double t = dsub(is[j], level[j]);
            trend[j] = dadd(dmul(beta, t), dmul(one_b, trend[j]));
            level[j] = dadd(dmul(alpha, is[j]), dmul(one_a, level[j]));
        }
    }
    if (lane == 0) p.partial[item] = sum;
}

// 4. H per theta and the first argmax.
__global__ __launch_bounds__(256) void finish_kernel(CalibParams p) {
    __shared__ double s_h[kMaxCalibGrid];
    for (int th = threadIdx.x; th < p.n; th += 256) {
        double s = 0.0;
        for (int c = 0; c < p.nchunks; ++c) s = dadd(s, p.partial[(size_t)th * p.nchunks + c]);
        const double h = p.rows > 1 ? s / (double)(p.rows - 1) : 0.0;
        p.H[th] = h;
        s_h[th] = h;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int best = 0;
        for (int th = 1; th < p.n; ++th)
            if (s_h[th] > s_h[best]) best = th;
        p.best[0] = best;
    }
}

int calib_chunks(int rows) { return rows > 1 ? (rows - 1 + kCalibChunk - 1) / kCalibChunk : 0; }

template <int KPL>
hipError_t launch_kpl(const CalibParams &p, hipStream_t stream) {
    if (p.rows > 1) {
        PRR_LAUNCH(rows_topk_kernel<KPL>, dim3((p.rows - 1 + 3) / 4), dim3(256), stream, p);
        PRR_LAUNCH(ema_chain_kernel, dim3((p.n * p.blocks + 255) / 256), dim3(256), stream, p);
        PRR_LAUNCH(replay_kernel<KPL>, dim3((p.n * p.nchunks + 3) / 4), dim3(256), stream, p);
    }
    PRR_LAUNCH(finish_kernel, dim3(1), dim3(256), stream, p);
    return hipGetLastError();
}

}  // namespace

size_t calib_workspace_bytes(int rows, int blocks, int n) {
    const size_t nch = (size_t)calib_chunks(rows);
    const size_t mask = ((size_t)rows * 64 * 4 + 255) / 256 * 256;
    const size_t ck = (size_t)n * std::max<size_t>(nch, 1) * 2 * blocks * sizeof(double);
    const size_t part = (size_t)n * std::max<size_t>(nch, 1) * sizeof(double);
    return mask + ck + part;
}

hipError_t launch_calibrate(const float *scores, int rows, int blocks, int k, const double *grid, int n,
                            double *H, int32_t *best, void *ws, hipStream_t stream) {
    CalibParams p;
    p.scores = scores;
    p.grid = grid;
    p.H = H;
    p.best = best;
    p.rows = rows;
    p.blocks = blocks;
    p.k = k;
    p.n = n;
    p.nchunks = calib_chunks(rows);
    const size_t mask = ((size_t)rows * 64 * 4 + 255) / 256 * 256;
    const size_t nch = std::max(p.nchunks, 1);
    p.amask = (uint32_t *)ws;
    p.ckpt = (double *)((char *)ws + mask);
    p.partial = p.ckpt + (size_t)n * nch * 2 * blocks;
    if (blocks <= 64) return launch_kpl<1>(p, stream);
    if (blocks <= 128) return launch_kpl<2>(p, stream);
    if (blocks <= 256) return launch_kpl<4>(p, stream);
    if (blocks <= 512) return launch_kpl<8>(p, stream);
    return launch_kpl<16>(p, stream);
}

}  // namespace prr
