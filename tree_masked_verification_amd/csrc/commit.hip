// commit.hip -- prefix-sharing path-index commit of the accepted K/V rows (gfx950).
//
// After acceptance the cache holds [prefix | tree rows in node-id order].  The accepted
// path's rows are compacted right behind the prefix, in depth order, in place; the
// prefix itself is never touched and rows that are already in place are not moved
// (EAGLE-Pangu, Chinese technical summary section 2.1: commit by path index with a
// prefix-sharing fast reorder that only moves the newly accepted segment).
//
// One workgroup per (layer, sequence) handles every KV head and both caches.  A source
// row can be another row's destination (ids need not be topological), so each pass
// first copies all moving source rows into LDS, waits at a barrier, then writes them to
// their destinations -- no row is read after it has been overwritten.  Rows move as
// 16-byte vectors.
//
// Paged caches (vLLM-style blocks, the PagedAttention-for-trees notes of the
// speculative-decoding survey page): logical slot t of sequence b lives in page
// table[b][t / page] at row t % page.  The same moves go through the block table.  Only
// the blocks that hold slots of [P, P + A) are ever written, a partial block at a time (a
// commit moves at most D_max rows per layer and head).  The evicting variant then
// rewrites the table: every block of the tree that now lies wholly at or beyond the new
// length -- a discarded branch's block -- is cleared and its page handed back to the
// caller's free list (the page's block eviction).
#include "tmv_device.hpp"

namespace {

constexpr int kCommitThreads = 256;
constexpr int kCommitLds = 64 * 1024;     // >= D_max * row bytes (host-checked)

// block table of a paged cache: page of logical slot t of sequence b is
// tab[b * stride + (t >> shift)], valid when in [0, npages)
struct CommitPages {
    const int32_t *tab;
    int64_t stride;
    int shift;
    int npages;
};

// PAGED: s_b is the page stride
template <bool PAGED>
__global__ void __launch_bounds__(kCommitThreads)
commit_kernel(int n_layers, int B, int Hkv, int row_bytes, int L_cap, int D_max,
              uint8_t *__restrict__ kc, uint8_t *__restrict__ vc,
              int64_t s_layer, int64_t s_b, int64_t s_h, int64_t s_t,      // bytes
              const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ n_nodes,
              const int32_t *__restrict__ accept_len, const int32_t *__restrict__ path,
              int32_t *__restrict__ status, int32_t *__restrict__ new_len, CommitPages pg)
{
    __shared__ uint4 snap[kCommitLds / 16];
    __shared__ int src_row[128], path_sh[128];
    __shared__ int64_t src_off[128], dst_off[128];   // byte offsets of the moving rows' slots
    __shared__ int wcount[kCommitThreads / 64];

    const int layer = blockIdx.x / B, b = blockIdx.x % B;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int P = prefix_len[b], M = n_nodes[b], A = accept_len[b];
    const int st = status[b];
    const int32_t *pth = path + static_cast<int64_t>(b) * D_max;
    if (tid < D_max) path_sh[tid] = pth[tid];            // the whole path in one round trip
    __syncthreads();

    // which path entries move (destination P + j, source P + path[j] - 1, j < A), compacted
    // in path order by a block scan: a ballot per wave, then the waves' counts
    const bool base_ok = st == TMV_OK && P >= 0 && static_cast<int64_t>(P) + M <= L_cap && A >= 0 && A <= D_max &&
                         A <= M;
    const int node = base_ok && tid < A ? path_sh[tid] : 1;
    const bool bad = base_ok && tid < A && (node < 1 || node > M);
    const bool mv = base_ok && tid < A && !bad && node - 1 != tid;
    const uint64_t bal = __ballot(mv);
    if (lane == 0) wcount[wv] = __popcll(bal);
    const bool fits = base_ok && __syncthreads_or(bad ? 1 : 0) == 0;
    int before = __popcll(bal & ((1ull << lane) - 1)), nmove = 0;
#pragma unroll
    for (int w = 0; w < kCommitThreads / 64; ++w) {
        before += w < wv ? wcount[w] : 0;
        nmove += wcount[w];
    }
    if (mv) src_row[before] = tid;
    if (!fits) nmove = 0;
    __syncthreads();
    // byte offsets of the moving rows' slots, one thread per row (paged: through the
    // block table; every page involved must be valid)
    bool bad_page = false;
    if (fits && tid < nmove) {
        const int j = src_row[tid];
        const int64_t src = static_cast<int64_t>(P) + path_sh[j] - 1, dst = static_cast<int64_t>(P) + j;
        if constexpr (PAGED) {
            const int32_t *trow = pg.tab + static_cast<int64_t>(b) * pg.stride;
            const int ps = trow[src >> pg.shift], pd = trow[dst >> pg.shift];
            bad_page = ps < 0 || ps >= pg.npages || pd < 0 || pd >= pg.npages;
            const int64_t mask = (int64_t(1) << pg.shift) - 1;
            src_off[tid] = (bad_page ? 0 : ps) * s_b + (src & mask) * s_t;
            dst_off[tid] = (bad_page ? 0 : pd) * s_b + (dst & mask) * s_t;
        } else {
            src_off[tid] = b * s_b + src * s_t;
            dst_off[tid] = b * s_b + dst * s_t;
        }
    }
    const bool rejected = __syncthreads_or(bad_page ? 1 : 0) != 0;
    const bool ok = fits && !rejected;
    if (tid == 0 && layer == 0) {
        new_len[b] = ok ? P + A : P;
        if (!ok && st == TMV_OK) status[b] = TMV_ERR_INPUT;
    }
    if (!ok || nmove == 0) return;

    const int n = nmove;
    const int segs = row_bytes / 16;
    const int units = 2 * Hkv;                               // (head, K|V)
    const int per_pass = max(1, (kCommitLds / 16) / (n * segs));
    for (int u0 = 0; u0 < units; u0 += per_pass) {
        const int u1 = min(units, u0 + per_pass);
        const int work = (u1 - u0) * n * segs;
        for (int e = tid; e < work; e += kCommitThreads) {
            const int uu = e / (n * segs), rem = e % (n * segs);
            const int r = rem / segs, sg = rem % segs;
            const int unit = u0 + uu, h = unit >> 1;
            const uint8_t *base = ((unit & 1) ? vc : kc) + layer * s_layer + h * s_h;
            snap[e] = *reinterpret_cast<const uint4 *>(base + src_off[r] + sg * 16);
        }
        __syncthreads();
        for (int e = tid; e < work; e += kCommitThreads) {
            const int uu = e / (n * segs), rem = e % (n * segs);
            const int r = rem / segs, sg = rem % segs;
            const int unit = u0 + uu, h = unit >> 1;
            uint8_t *base = ((unit & 1) ? vc : kc) + layer * s_layer + h * s_h;
            *reinterpret_cast<uint4 *>(base + dst_off[r] + sg * 16) = snap[e];
        }
        __syncthreads();
    }
}

// Block eviction after a paged commit (ordered after it on the stream, so every layer's
// row moves, which may read rows of these blocks, are done): one workgroup per sequence;
// the blocks of the tree's slots [P, P + M) that start at or beyond new_len are cleared
// in the table and their pages appended to the free list.  A full list keeps the block.
__global__ void __launch_bounds__(64)
evict_kernel(int M_max, int page_shift, int max_blocks, int npages, int32_t *__restrict__ tab, int64_t stride,
             const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ n_nodes,
             const int32_t *__restrict__ status, const int32_t *__restrict__ new_len,
             int32_t *__restrict__ freed, int32_t *__restrict__ freed_count, int capacity)
{
    const int b = blockIdx.x;
    if (status[b] != TMV_OK) return;
    const int P = prefix_len[b], M = n_nodes[b], nl = new_len[b];
    if (P < 0 || M < 0 || M > M_max || nl < P) return;
    const int ps = 1 << page_shift;
    const int64_t end = static_cast<int64_t>(P) + M;          // first slot past the tree
    const int first = (nl + ps - 1) >> page_shift;            // first block wholly >= new_len
    const int64_t last = (end + ps - 1) >> page_shift;        // one past the tree's last block
    int32_t *trow = tab + static_cast<int64_t>(b) * stride;
    for (int64_t i = first + threadIdx.x; i < last && i < max_blocks; i += 64) {
        const int pg = trow[i];
        if (pg < 0 || pg >= npages) continue;
        const int slot = atomicAdd(freed_count, 1);
        if (slot >= capacity) continue;                        // no room: the block stays
        freed[slot] = pg;
        trow[i] = -1;
    }
}

}  // namespace

extern "C" int tmv_kv_commit_path(int dtype, int n_layers, int B, int Hkv, int d, int L_cap,
                                  int M_max, int D_max,
                                  void *k_cache, void *v_cache, const int64_t *kv_stride,
                                  const int32_t *prefix_len, const int32_t *n_nodes,
                                  const int32_t *accept_len, const int32_t *path,
                                  int32_t *status, int32_t *new_len, void *stream)
{
    if (dtype != TMV_F32 && dtype != TMV_BF16) return TMV_ERR_ARG;
    const int es = dtype == TMV_F32 ? 4 : 2;
    if (n_layers < 0 || B < 0 || Hkv <= 0 || d <= 0 || L_cap < 0) return TMV_ERR_ARG;
    if (M_max < 0 || M_max > 128 || D_max < 0 || D_max > 128) return TMV_ERR_ARG;
    const int row_bytes = d * es;
    if (row_bytes % 16 != 0 || row_bytes > 512) return TMV_ERR_ARG;
    if (!kv_stride) return TMV_ERR_ARG;
    if (B == 0) return TMV_OK;
    if (!prefix_len || !n_nodes || !accept_len || !status || !new_len || (D_max > 0 && !path)) return TMV_ERR_ARG;
    if (n_layers > 0 && (!k_cache || !v_cache)) return TMV_ERR_ARG;
    for (int i = 0; i < 4; ++i)
        if (kv_stride[i] < 0 || (kv_stride[i] * es) % 16 != 0) return TMV_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15u) return TMV_ERR_ARG;
    // new_len and the status checks are written by the layer-0 workgroups: with no
    // layers, one pass over the sequences still publishes them (and moves no rows)
    const int layers = n_layers > 0 ? n_layers : 1;
    const int64_t blocks = static_cast<int64_t>(layers) * B;
    if (blocks > 0x7fffffff) return TMV_ERR_ARG;
    hipLaunchKernelGGL(commit_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kCommitThreads), 0,
                       static_cast<hipStream_t>(stream), layers, B, n_layers > 0 ? Hkv : 0, row_bytes, L_cap, D_max,
                       static_cast<uint8_t *>(k_cache), static_cast<uint8_t *>(v_cache),
                       kv_stride[0] * es, kv_stride[1] * es, kv_stride[2] * es, kv_stride[3] * es,
                       prefix_len, n_nodes, accept_len, path, status, new_len, CommitPages{nullptr, 0, 0, 0});
    return tmv_host::launch_status(hipGetLastError());
}

extern "C" int tmv_kv_commit_path_paged(int dtype, int n_layers, int B, int Hkv, int d, int num_pages, int page_size,
                                        const int32_t *block_table, int64_t table_stride, int max_blocks,
                                        int M_max, int D_max, void *k_pages, void *v_pages,
                                        const int64_t *page_stride, const int32_t *prefix_len,
                                        const int32_t *n_nodes, const int32_t *accept_len, const int32_t *path,
                                        int32_t *status, int32_t *new_len, void *stream)
{
    if (dtype != TMV_F32 && dtype != TMV_BF16) return TMV_ERR_ARG;
    const int es = dtype == TMV_F32 ? 4 : 2;
    if (n_layers < 0 || B < 0 || Hkv <= 0 || d <= 0 || num_pages < 1) return TMV_ERR_ARG;
    if (page_size < 1 || (page_size & (page_size - 1)) || page_size > (1 << 20)) return TMV_ERR_ARG;
    if (max_blocks < 1 || table_stride < max_blocks) return TMV_ERR_ARG;
    const int64_t L_cap = static_cast<int64_t>(page_size) * max_blocks;
    if (L_cap > 0x7fffffff) return TMV_ERR_ARG;
    if (M_max < 0 || M_max > 128 || D_max < 0 || D_max > 128) return TMV_ERR_ARG;
    const int row_bytes = d * es;
    if (row_bytes % 16 != 0 || row_bytes > 512) return TMV_ERR_ARG;
    if (!page_stride) return TMV_ERR_ARG;
    if (B == 0) return TMV_OK;
    if (!block_table || !prefix_len || !n_nodes || !accept_len || !status || !new_len || (D_max > 0 && !path))
        return TMV_ERR_ARG;
    if (n_layers > 0 && (!k_pages || !v_pages)) return TMV_ERR_ARG;
    for (int i = 0; i < 4; ++i)
        if (page_stride[i] < 0 || (page_stride[i] * es) % 16 != 0) return TMV_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages)) & 15u) return TMV_ERR_ARG;
    const int layers = n_layers > 0 ? n_layers : 1;
    const int64_t blocks = static_cast<int64_t>(layers) * B;
    if (blocks > 0x7fffffff) return TMV_ERR_ARG;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    hipLaunchKernelGGL(commit_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kCommitThreads), 0,
                       static_cast<hipStream_t>(stream), layers, B, n_layers > 0 ? Hkv : 0, row_bytes,
                       static_cast<int>(L_cap), D_max, static_cast<uint8_t *>(k_pages), static_cast<uint8_t *>(v_pages),
                       page_stride[0] * es, page_stride[1] * es, page_stride[2] * es, page_stride[3] * es,
                       prefix_len, n_nodes, accept_len, path, status, new_len,
                       CommitPages{block_table, table_stride, shift, num_pages});
    return tmv_host::launch_status(hipGetLastError());
}

extern "C" int tmv_kv_commit_path_paged_evict(int dtype, int n_layers, int B, int Hkv, int d, int num_pages,
                                              int page_size, int32_t *block_table, int64_t table_stride,
                                              int max_blocks, int M_max, int D_max, void *k_pages, void *v_pages,
                                              const int64_t *page_stride, const int32_t *prefix_len,
                                              const int32_t *n_nodes, const int32_t *accept_len, const int32_t *path,
                                              int32_t *status, int32_t *new_len, int32_t *freed_pages,
                                              int32_t *freed_count, int freed_capacity, void *stream)
{
    if (freed_capacity < 0 || (B > 0 && (!freed_pages || !freed_count))) return TMV_ERR_ARG;
    const int rc = tmv_kv_commit_path_paged(dtype, n_layers, B, Hkv, d, num_pages, page_size, block_table,
                                            table_stride, max_blocks, M_max, D_max, k_pages, v_pages, page_stride,
                                            prefix_len, n_nodes, accept_len, path, status, new_len, stream);
    if (rc != TMV_OK || B == 0) return rc;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    hipLaunchKernelGGL(evict_kernel, dim3(B), dim3(64), 0, static_cast<hipStream_t>(stream), M_max, shift, max_blocks,
                       num_pages, block_table, table_stride, prefix_len, n_nodes, status, new_len, freed_pages,
                       freed_count, freed_capacity);
    return tmv_host::launch_status(hipGetLastError());
}
