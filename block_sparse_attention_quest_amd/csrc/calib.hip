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
// top-K sets of different rows are independent.  A row is held by one workgroup of W waves (W = 1 up to
// 1024 blocks, 2 up to 2048, 4 up to 4096; up to 16 blocks per thread).  Four launches:
//   1. rows_topk:  one workgroup per row, A_phi as a bit mask (the top-K kernels' radix select);
//   2. ema_chain:  one thread per (theta, block) runs the recurrence over all rows and stores the state
//                  at the start of every chunk of kChunk rows (checkpoints);
//   3. replay:     one workgroup per (theta, chunk) resumes from its checkpoint with the same operations,
//                  predicts, selects P_phi, and sums h over its rows;
//   4. finish:     H = sum of the chunk sums / (rows - 1) per theta, and the first argmax.
// Top-K ties go to the smaller block index; hit-rate sums use the same reduction tree for numerator
// and denominator, so P = A gives h = 1 exactly.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "prr_internal.hpp"
#include "select_core.hpp"   // float64 helpers and the exact radix select (contraction off)

#pragma clang fp contract(off)

namespace prr {
namespace {

constexpr int kCalibChunk = 64;   // rows per replay workgroup

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = dadd(v, __shfl_xor(v, o));
    return v;
}

// Sums of x and y over the workgroup's W waves with the same reduction tree for both (a butterfly in
// each wave, then the waves' sums in wave order), so equal inputs give equal sums.
template <int W>
__device__ __forceinline__ void block_sum2_f64(double &x, double &y, double (&s_part)[2][W]) {
    x = wave_sum_f64(x);
    y = wave_sum_f64(y);
    if constexpr (W > 1) {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
            s_part[0][wave] = x;
            s_part[1][wave] = y;
        }
        __syncthreads();
        x = 0.0;
        y = 0.0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            x = dadd(x, s_part[0][w]);
            y = dadd(y, s_part[1][w]);
        }
        __syncthreads();
    }
}

struct CalibParams {
    const float *scores;    // [rows][blocks]
    const double *grid;     // [n][3]: alpha, beta, gamma
    double *H;              // [n]
    int32_t *best;          // [1]
    uint32_t *amask;        // [rows][64 W]: thread t's KPT-bit share of A_phi (blocks t KPT .. + KPT)
    double *ckpt;           // [n][nchunks][2][blocks]: level, trend at the start of each chunk
    double *partial;        // [n][nchunks]
    int rows, blocks, k, n, nchunks;
};

// 1. A_phi = top-k of row phi (phi >= 1), one workgroup of W waves per row.
template <int KPT, int W>
__global__ __launch_bounds__(64 * W) void rows_topk_kernel(CalibParams p) {
    __shared__ TopkSmem<W> sm;
    const int phi = 1 + blockIdx.x;
    const float *row = p.scores + (size_t)phi * p.blocks;
    uint64_t key[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int b = threadIdx.x * KPT + j;
        key[j] = b < p.blocks ? order_key((double)row[b]) : 0ull;
    }
    const uint32_t sel = block_topk<KPT, W>(key, p.blocks, p.k, sm);
    p.amask[(size_t)phi * (64 * W) + threadIdx.x] = sel;
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
    // Rows in groups of kRowGroup, double-buffered: the next group's scores (independent of the
    // recurrence) load while the current group is absorbed in row order.  The launch has fewer waves than
    // the GPU has SIMDs, so these loads in flight are what hides the memory latency (8192 x 512 scores,
    // 80 candidates: 3.96 ms for the whole calibration with one load per row, 2.26 ms grouped).
    constexpr int kRowGroup = 16;   // 16, 32 and 64 rows measured within 10% of each other; 16 takes fewest registers
    float cur[kRowGroup], nxt[kRowGroup];
    auto load_group = [&](int phi0, float (&v)[kRowGroup]) {
#pragma unroll
        for (int i = 0; i < kRowGroup; ++i)
            v[i] = phi0 + i < p.rows ? p.scores[(size_t)(phi0 + i) * p.blocks + b] : 0.0f;
    };
    load_group(1, cur);
    for (int phi0 = 1; phi0 < p.rows; phi0 += kRowGroup) {
        if (phi0 + kRowGroup < p.rows) load_group(phi0 + kRowGroup, nxt);
#pragma unroll
        for (int i = 0; i < kRowGroup; ++i) {
            const int phi = phi0 + i;
            if (phi < p.rows) {
                const double is = (double)cur[i];
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
#pragma unroll
        for (int i = 0; i < kRowGroup; ++i) cur[i] = nxt[i];
    }
}

// 3. One workgroup per (theta, chunk): predict, select P_phi, score-weighted hit rate, absorb the row.
template <int KPT, int W>
__global__ __launch_bounds__(64 * W) void replay_kernel(CalibParams p) {
    __shared__ TopkSmem<W> sm;
    __shared__ double s_part[2][W];
    const int item = blockIdx.x;
    const int th = item / p.nchunks, c = item - th * p.nchunks;
    const double alpha = p.grid[3 * th], beta = p.grid[3 * th + 1], gamma = p.grid[3 * th + 2];
    const double one_a = dsub(1.0, alpha), one_b = dsub(1.0, beta);
    const double *ck = p.ckpt + ((size_t)th * p.nchunks + c) * 2 * p.blocks;
    const int base = threadIdx.x * KPT;
    double level[KPT], trend[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int b = min(base + j, p.blocks - 1);
        level[j] = ck[b];
        trend[j] = ck[p.blocks + b];
    }
    const int phi0 = 1 + c * kCalibChunk;
    const int phi1 = min(p.rows, phi0 + kCalibChunk);
    // the row's true-set mask and scores, loaded one row ahead of their use
    auto load_row = [&](int phi, uint32_t &am, float (&v)[KPT]) {
        am = p.amask[(size_t)phi * (64 * W) + threadIdx.x];
        const float *row = p.scores + (size_t)phi * p.blocks;
#pragma unroll
        for (int j = 0; j < KPT; ++j) v[j] = base + j < p.blocks ? row[base + j] : 0.0f;
    };
    uint32_t am_next;
    float v_next[KPT];
    load_row(phi0, am_next, v_next);
    double sum = 0.0;
    for (int phi = phi0; phi < phi1; ++phi) {
        const uint32_t am = am_next;
        float v[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) v[j] = v_next[j];
        if (phi + 1 < phi1) load_row(phi + 1, am_next, v_next);
        uint64_t key[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = order_key(dadd(level[j], dmul(gamma, trend[j])));   // prediction
        __syncthreads();   // the previous row's selection scratch is free
        const uint32_t pm = block_topk<KPT, W>(key, p.blocks, p.k, sm);
        double is[KPT];
        double num = 0.0, den = 0.0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            is[j] = (double)v[j];
            if (am >> j & 1u) {
                den = dadd(den, is[j]);
                num = dadd(num, (pm >> j & 1u) ? is[j] : 0.0);
            }
        }
        block_sum2_f64<W>(num, den, s_part);
        sum = dadd(sum, den != 0.0 ? num / den : 0.0);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const double t = dsub(is[j], level[j]);
            trend[j] = dadd(dmul(beta, t), dmul(one_b, trend[j]));
            level[j] = dadd(dmul(alpha, is[j]), dmul(one_a, level[j]));
        }
    }
    if (threadIdx.x == 0) p.partial[item] = sum;
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

// Waves per row: one up to 1024 blocks (16 per lane), then as many as 16 blocks per thread need.
int calib_waves(int blocks) { return blocks <= 1024 ? 1 : blocks <= 2048 ? 2 : 4; }

size_t mask_bytes(int rows, int blocks) {
    return ((size_t)rows * 64 * calib_waves(blocks) * 4 + 255) / 256 * 256;
}

template <int KPT, int W>
hipError_t launch_shape(const CalibParams &p, hipStream_t stream) {
    if (p.rows > 1) {
        PRR_LAUNCH(rows_topk_kernel<KPT, W>, dim3(p.rows - 1), dim3(64 * W), stream, p);
        PRR_LAUNCH(ema_chain_kernel, dim3((p.n * p.blocks + 255) / 256), dim3(256), stream, p);
        PRR_LAUNCH(replay_kernel<KPT, W>, dim3(p.n * p.nchunks), dim3(64 * W), stream, p);
    }
    PRR_LAUNCH(finish_kernel, dim3(1), dim3(256), stream, p);
    return hipGetLastError();
}

}  // namespace

size_t calib_workspace_bytes(int rows, int blocks, int n) {
    const size_t nch = (size_t)calib_chunks(rows);
    const size_t ck = (size_t)n * std::max<size_t>(nch, 1) * 2 * blocks * sizeof(double);
    const size_t part = (size_t)n * std::max<size_t>(nch, 1) * sizeof(double);
    return mask_bytes(rows, blocks) + ck + part;
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
    const size_t nch = std::max(p.nchunks, 1);
    p.amask = (uint32_t *)ws;
    p.ckpt = (double *)((char *)ws + mask_bytes(rows, blocks));
    p.partial = p.ckpt + (size_t)n * nch * 2 * blocks;
    if (blocks <= 64) return launch_shape<1, 1>(p, stream);
    if (blocks <= 128) return launch_shape<2, 1>(p, stream);
    if (blocks <= 256) return launch_shape<4, 1>(p, stream);
    if (blocks <= 512) return launch_shape<8, 1>(p, stream);
    if (blocks <= 1024) return launch_shape<16, 1>(p, stream);
    if (blocks <= 2048) return launch_shape<16, 2>(p, stream);
    return launch_shape<16, 4>(p, stream);
}

}  // namespace prr
