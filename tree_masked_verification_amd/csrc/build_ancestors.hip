// build_ancestors.hip -- accelerator-safe tree tensors on the device.
//
// Parent pointers are remapped onto a virtual root row 0 and expanded into an ancestor
// table whose every entry lies in [0, M_b]; range, acyclicity, depth and validity-closure
// checks yield a per-sequence status, and a failed sequence's rows are cleared.
// (EAGLE-Pangu, Chinese technical summary section 2.2; Portuguese summary section 2.)
//
// One workgroup per sequence, one thread per node row.  The parent table of the sequence
// is staged in LDS, so each walk (at most M_b hops) touches only LDS; anc rows are
// written as the walk goes.  The status is the smallest nonzero code of any node,
// reduced with an LDS atomic.
#include "tmv_device.hpp"

namespace {

constexpr int kBuildThreads = 256;      // >= M_max + 1 (M_max <= 128)

__global__ void __launch_bounds__(kBuildThreads)
build_ancestors_kernel(int M_max, int D_max, int parent_format,
                       const int32_t *__restrict__ parents, const uint8_t *__restrict__ valid,
                       const int32_t *__restrict__ n_nodes,
                       int32_t *__restrict__ anc, int32_t *__restrict__ depth,
                       int32_t *__restrict__ status)
{
    __shared__ int32_t par[kBuildThreads];
    __shared__ uint8_t ok[kBuildThreads];
    __shared__ int32_t worst;                 // smallest nonzero code, or INT_MAX

    const int b = blockIdx.x, i = threadIdx.x;
    const int R = M_max + 1, W = D_max + 1;
    const int M = n_nodes[b];
    const bool m_ok = M >= 0 && M <= M_max;
    int32_t *arow = anc + (static_cast<int64_t>(b) * R + i) * W;

    if (i == 0) worst = m_ok ? 0x7fffffff : TMV_ERR_RANGE;
    if (m_ok && i >= 1 && i <= M) {
        int p;
        if (parent_format == TMV_PARENTS_VROOT) {
            p = parents[static_cast<int64_t>(b) * R + i];
        } else {
            const int raw = parents[static_cast<int64_t>(b) * M_max + (i - 1)];
            p = raw == -1 ? 0 : (raw < -1 ? -1 : raw + 1);
        }
        par[i] = p;
        ok[i] = valid ? (valid[static_cast<int64_t>(b) * R + i] != 0) : 1;
    }
    __syncthreads();

    int d = 0, code = TMV_OK;
    if (i < R) {
        int written = 0;
        if (m_ok && i >= 1 && i <= M && ok[i]) {
            int h = i, k = 0;
            for (;;) {
                if (k <= D_max) { arow[k] = h; written = k + 1; }
                const int p = par[h];
                if (p < 0 || p > M) { code = TMV_ERR_RANGE; break; }
                if (p == 0) { d = k + 1; break; }
                if (!ok[p]) { code = TMV_ERR_CLOSURE; break; }
                h = p;
                if (++k >= M) { code = TMV_ERR_CYCLE; break; }   // M hops without the root
            }
            if (code == TMV_OK && d > D_max) code = TMV_ERR_DEPTH;
        }
        for (int k = written; k < W; ++k) arow[k] = 0;
        if (code != TMV_OK) atomicMin(&worst, code);
    }
    __syncthreads();

    const int st = worst == 0x7fffffff ? TMV_OK : worst;
    if (i < R) {
        if (st != TMV_OK) {
            for (int k = 0; k < W; ++k) arow[k] = 0;
            d = 0;
        }
        depth[static_cast<int64_t>(b) * R + i] = d;
    }
    if (i == 0) status[b] = st;
}

}  // namespace

extern "C" int tmv_tree_build_ancestors(int B, int M_max, int D_max, int parent_format,
                                        const int32_t *parents, const uint8_t *valid,
                                        const int32_t *n_nodes,
                                        int32_t *anc, int32_t *depth, int32_t *status,
                                        void *stream)
{
    if (B < 0 || M_max < 0 || M_max > 128 || D_max < 0 || D_max > 128) return TMV_ERR_ARG;
    if (parent_format != TMV_PARENTS_VROOT && parent_format != TMV_PARENTS_NEG1) return TMV_ERR_ARG;
    if (B == 0) return TMV_OK;
    if (!n_nodes || !anc || !depth || !status || (M_max > 0 && !parents)) return TMV_ERR_ARG;
    hipLaunchKernelGGL(build_ancestors_kernel, dim3(B), dim3(kBuildThreads), 0,
                       static_cast<hipStream_t>(stream), M_max, D_max, parent_format, parents, valid,
                       n_nodes, anc, depth, status);
    return tmv_host::launch_status(hipGetLastError());
}
