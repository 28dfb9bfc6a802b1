// accept.hip -- choosing the accepted path of a verified draft tree (gfx950).
//
// GREEDY: the teacher's argmax of every live row, then the deepest node whose whole
//   path matches those choices (Medusa section of "Speculative Decoding Hierarquico":
//   the longest valid branch is kept).  The row scans are the HBM-bound part: one
//   workgroup per (sequence, row, vocabulary chunk) reads its chunk with 16-byte loads
//   and reduces a 64-bit key (order-preserving value bits << 32 | ~index), so max() gives
//   the largest value and, on ties, the smallest index.  A second kernel (one
//   workgroup per sequence, ordered after the scan on the stream) merges the chunk keys
//   and picks the path -- no cross-workgroup synchronisation inside a kernel.
// SAMPLE: modified rejection sampling (same page, its rejection-sampling section and
//   FAQ), children of the current node tried in ascending id against the running
//   residual.  Exact integer fixed point, so the result is bit-identical to any correct
//   implementation: one workgroup walks one sequence; every full-row pass (row sums,
//   residual update, inverse-CDF draw) is a block-wide integer reduction or scan.
#include "tmv_device.hpp"

namespace {

using tmv::kWave;
using tmv::u128;

// ============================================================== greedy
constexpr int kScanThreads = 256;
constexpr int kScanChunk = 4096;          // vocabulary entries per workgroup (four 16-byte loads per thread)
constexpr uint64_t kNanKey = ~0ull;       // a chunk with a NaN reports the all-ones key

__device__ __forceinline__ uint32_t order_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void scan_one(float v, int idx, uint64_t &best, bool &nan) {
    if (v != v) nan = true;
    const uint64_t key = (static_cast<uint64_t>(order_bits(v)) << 32) | (0xffffffffu - static_cast<uint32_t>(idx));
    best = key > best ? key : best;
}

template <int DT>
__global__ void __launch_bounds__(kScanThreads)
greedy_scan_kernel(int M_max, int V, int nchunk, const void *__restrict__ teacher, int64_t sb, int64_t sr,
                   const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ depth,
                   const int32_t *__restrict__ status, uint64_t *__restrict__ keys)
{
    __shared__ uint64_t red[kScanThreads / kWave];
    const int R = M_max + 1;
    const int chunk = blockIdx.x % nchunk;
    const int u = (blockIdx.x / nchunk) % R;
    const int b = blockIdx.x / (nchunk * R);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    // The row's loads go out before the words that decide whether the row is live have
    // returned: every (b, u, chunk) of the grid addresses the teacher tensor in bounds, so
    // a dead row only costs bandwidth, and a live one saves a round trip.
    const int M = n_nodes[b];
    const int st = status[b];
    const int dp = u > 0 ? depth[static_cast<int64_t>(b) * R + u] : 1;

    const int x0 = chunk * kScanChunk;
    const int x1 = min(V, x0 + kScanChunk);
    uint64_t best = 0;
    bool nan = false;
    if constexpr (DT == TMV_F32) {
        const float *row = static_cast<const float *>(teacher) + b * sb + static_cast<int64_t>(u) * sr;
        constexpr int kPer = kScanChunk / (4 * kScanThreads);        // float4 per thread
        if (x1 - x0 == kScanChunk && ((reinterpret_cast<uintptr_t>(row + x0) & 15u) == 0)) {
            const float4 *r4 = reinterpret_cast<const float4 *>(row + x0);
            float4 f[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) f[i] = r4[tid + i * kScanThreads];
            if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int x = x0 + 4 * (tid + i * kScanThreads);
                scan_one(f[i].x, x, best, nan);
                scan_one(f[i].y, x + 1, best, nan);
                scan_one(f[i].z, x + 2, best, nan);
                scan_one(f[i].w, x + 3, best, nan);
            }
        } else {
            if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
            for (int x = x0 + tid; x < x1; x += kScanThreads) scan_one(row[x], x, best, nan);
        }
    } else {
        const uint16_t *row = static_cast<const uint16_t *>(teacher) + b * sb + static_cast<int64_t>(u) * sr;
        constexpr int kPer = kScanChunk / (8 * kScanThreads);        // 8 bf16 per thread and load
        if (x1 - x0 == kScanChunk && ((reinterpret_cast<uintptr_t>(row + x0) & 15u) == 0)) {
            const uint4 *r8 = reinterpret_cast<const uint4 *>(row + x0);
            uint4 h[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) h[i] = r8[tid + i * kScanThreads];
            if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int x = x0 + 8 * (tid + i * kScanThreads);
                const uint32_t w[4] = {h[i].x, h[i].y, h[i].z, h[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    scan_one(__uint_as_float(w[e] << 16), x + 2 * e, best, nan);
                    scan_one(__uint_as_float(w[e] & 0xffff0000u), x + 2 * e + 1, best, nan);
                }
            }
        } else {
            if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
            for (int x = x0 + tid; x < x1; x += kScanThreads) scan_one(tmv::bf16_to_f32(row[x]), x, best, nan);
        }
    }
    if (nan) best = kNanKey;
    best = tmv::wave_max_u64(best);
    if (lane == 0) red[wv] = best;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = red[0];
        for (int w = 1; w < kScanThreads / kWave; ++w) k = red[w] > k ? red[w] : k;
        keys[(static_cast<int64_t>(b) * R + u) * nchunk + chunk] = k;
    }
}

// One workgroup per sequence, after the scan: merge the chunk keys of every live row into
// t(u), check the draft tokens, mark matching nodes and pick the deepest (smallest id).
__global__ void __launch_bounds__(kScanThreads)
greedy_select_kernel(int M_max, int D_max, int V, int nchunk, const int32_t *__restrict__ tokens,
                     const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ anc,
                     const int32_t *__restrict__ depth, int32_t *__restrict__ status,
                     int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                     int32_t *__restrict__ next_token, const uint64_t *__restrict__ keys)
{
    constexpr int kKeyBatch = 32;                  // chunk keys per row fetched at once
    constexpr int kAncBatch = 8;                   // ancestor entries per node fetched at once
    __shared__ int32_t tsel[129], tok_sh[129];
    __shared__ int bad;
    __shared__ uint64_t best_node[kScanThreads / kWave];
    const int R = M_max + 1, W = D_max + 1;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;

    // one round trip: sequence scalars, this thread's row of keys, token, depth and
    // first ancestor entries (indices clamped into the tables)
    const int M = n_nodes[b];
    const int st_in = status[b];
    const int row = tid < R ? tid : R - 1;
    const int64_t rb = static_cast<int64_t>(b) * R + row;
    uint64_t kb[kKeyBatch];
#pragma unroll
    for (int c = 0; c < kKeyBatch; ++c) kb[c] = c < nchunk ? keys[rb * nchunk + c] : 0;
    const int tok = tokens[rb];
    const int dep = row > 0 ? depth[rb] : 0;
    int a8[kAncBatch];
    const int32_t *arow = anc + rb * W;
#pragma unroll
    for (int k = 0; k < kAncBatch; ++k) a8[k] = arow[k < W ? k : W - 1];

    // a node count outside [0, M_max] cannot come with an OK status from the build stage;
    // it is rejected here so that no row beyond the tables is ever addressed
    const int st = (st_in == TMV_OK && (M < 0 || M > M_max)) ? TMV_ERR_INPUT : st_in;
    int32_t *pth = path + static_cast<int64_t>(b) * D_max;
    if (tid == 0) bad = st != TMV_OK;
    if (tid < R) tok_sh[tid] = tok;
    __syncthreads();
    const bool row_live = st == TMV_OK && tid < R && tid <= M && (tid == 0 || dep >= 1);
    if (row_live) {
        uint64_t k = 0;
#pragma unroll
        for (int c = 0; c < kKeyBatch; ++c) k = kb[c] > k ? kb[c] : k;
        for (int c = kKeyBatch; c < nchunk; ++c) {
            const uint64_t kc = keys[rb * nchunk + c];
            k = kc > k ? kc : k;
        }
        if (k == kNanKey) bad = 1;
        tsel[tid] = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(k & 0xffffffffu));
        if (tid > 0 && (tok < 0 || tok >= V)) bad = 1;
    }
    __syncthreads();
    if (bad) {
        for (int j = tid; j < D_max; j += kScanThreads) pth[j] = 0;
        if (tid == 0) {
            accept_len[b] = 0;
            next_token[b] = 0;
            if (st_in == TMV_OK) status[b] = TMV_ERR_INPUT;
        }
        return;
    }
    // node i matches iff every node c on its path has token == t(parent(c)); the chosen
    // node maximises (depth, -id): key = depth << 8 | (255 - id)
    uint64_t key = 0;
    if (tid >= 1 && tid <= M && dep >= 1) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < kAncBatch; ++k) {
            if (k < dep) {
                const int parent = k + 1 < kAncBatch ? a8[k + 1] : arow[k + 1];
                ok = ok && tok_sh[a8[k]] == tsel[k + 1 < dep ? parent : 0];
            }
        }
        for (int k = kAncBatch; k < dep && ok; ++k)
            ok = tok_sh[arow[k]] == tsel[arow[k + 1]];
        if (ok) key = (static_cast<uint64_t>(dep) << 8) | static_cast<uint64_t>(255 - tid);
    }
    key = tmv::wave_max_u64(key);
    if (lane == 0) best_node[wv] = key;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = best_node[0];
        for (int w = 1; w < kScanThreads / kWave; ++w) k = best_node[w] > k ? best_node[w] : k;
        const int star = k ? 255 - static_cast<int>(k & 255u) : 0;
        const int dstar = static_cast<int>(k >> 8);
        best_node[0] = (static_cast<uint64_t>(dstar) << 32) | static_cast<uint32_t>(star);
        accept_len[b] = dstar;
        next_token[b] = tsel[star];
    }
    __syncthreads();
    const int dstar = static_cast<int>(best_node[0] >> 32), star = static_cast<int>(best_node[0] & 0xffffffffu);
    for (int j = tid; j < D_max; j += kScanThreads)
        pth[j] = j < dstar ? anc[(static_cast<int64_t>(b) * R + star) * W + (dstar - 1 - j)] : 0;
}

// ============================================================== sampling
constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;

// block-wide exact sum of one u128 per thread (result broadcast to every thread)
__device__ u128 block_sum_u128(u128 v, u128 *sh) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    v = tmv::wave_sum_u128(v);
    __syncthreads();
    if (lane == 0) sh[wv] = v;
    __syncthreads();
    u128 t = 0;
    for (int w = 0; w < kSampleWaves; ++w) t += sh[w];
    return t;
}

__device__ int block_or(int v, int *sh) {
    __syncthreads();
    if (threadIdx.x == 0) *sh = 0;
    __syncthreads();
    if (v) atomicOr(sh, 1);
    __syncthreads();
    return *sh;
}

// floor(p * 2^32) for p in [0,1] (exact: p * 2^32 is exact in fp64); flags bad entries
__device__ __forceinline__ uint64_t quantise(float p, int &bad) {
    if (!(p >= 0.f && p <= 1.f)) { bad = 1; return 0; }
    return static_cast<uint64_t>(static_cast<double>(p) * 4294967296.0);
}

struct Dist {       // the working distribution W of the walk
    const float *row;    // W(x) = floor(row[x] * 2^32) >> shift when stored == false
    int shift;
    bool stored;         // W lives in the workspace array
    u128 S;
};

__device__ __forceinline__ uint64_t dist_at(const Dist &D, const uint64_t *w, int x, int &bad) {
    if (D.stored) return w[x];
    return quantise(D.row[x], bad) >> D.shift;
}

__global__ void __launch_bounds__(kSampleThreads)
sample_walk_kernel(int M_max, int D_max, int V,
                   const int32_t *__restrict__ tokens,
                   const float *__restrict__ p, int64_t psb, int64_t psr,
                   const float *__restrict__ q, int64_t qsb, int64_t qsr,
                   uint64_t seed, uint64_t step,
                   const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ anc,
                   const int32_t *__restrict__ depth, int32_t *__restrict__ status,
                   int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                   int32_t *__restrict__ next_token, uint64_t *__restrict__ wsW)
{
    __shared__ u128 sh128[kSampleWaves];
    __shared__ int shflag;
    __shared__ int kids[129];
    __shared__ int nkids;
    __shared__ uint64_t shx[2];
    __shared__ int draw_tok;

    const int b = blockIdx.x, tid = threadIdx.x;
    const int R = M_max + 1, W = D_max + 1;
    const int M = n_nodes[b];
    int32_t *pth = path + static_cast<int64_t>(b) * D_max;
    uint64_t *w = wsW + static_cast<int64_t>(b) * V;
    const int st_in = status[b];
    const int st = (st_in == TMV_OK && (M < 0 || M > M_max)) ? TMV_ERR_INPUT : st_in;
    const uint64_t stream = (step << 32) | static_cast<uint32_t>(b);

    auto finish = [&](int code, int acc, int tok) {
        __syncthreads();
        if (code != TMV_OK) { acc = 0; tok = 0; }
        for (int j = tid; j < D_max; j += kSampleThreads)
            if (code != TMV_OK || j >= acc) pth[j] = 0;
        if (tid == 0) {
            accept_len[b] = acc;
            next_token[b] = tok;
            if (code != TMV_OK && st_in == TMV_OK) status[b] = code;
        }
    };
    if (st != TMV_OK) { finish(st, 0, 0); return; }

    // live tokens in range
    int bad = 0;
    for (int i = tid + 1; i <= M; i += kSampleThreads)
        if (depth[static_cast<int64_t>(b) * R + i] >= 1) {
            const int t = tokens[static_cast<int64_t>(b) * R + i];
            if (t < 0 || t >= V) bad = 1;
        }
    if (block_or(bad, &shflag)) { finish(TMV_ERR_INPUT, 0, 0); return; }

    // load (W, S) = quantised p row `row`, renormalised to <= 48 bits
    auto load_p = [&](int row, Dist &Dd) -> bool {
        const float *pr = p + b * psb + static_cast<int64_t>(row) * psr;
        int bd = 0;
        u128 s = 0;
        for (int x = tid; x < V; x += kSampleThreads) s += quantise(pr[x], bd);
        if (block_or(bd, &shflag)) return false;
        s = block_sum_u128(s, sh128);
        if (s == 0) return false;
        Dd.row = pr; Dd.shift = 0; Dd.stored = false; Dd.S = s;
        const int bl = tmv::bitlen_u128(s);
        if (bl > 48) {
            Dd.shift = bl - 48;
            u128 s2 = 0;
            for (int x = tid; x < V; x += kSampleThreads) s2 += quantise(pr[x], bd) >> Dd.shift;
            Dd.S = block_sum_u128(s2, sh128);
        }
        return true;
    };

    Dist cur;
    if (!load_p(0, cur)) { finish(TMV_ERR_INPUT, 0, 0); return; }
    uint64_t n = 0;           // draws consumed
    int u = 0, acc = 0;
    for (;;) {
        // children of u in ascending id
        __syncthreads();
        if (tid == 0) {
            int k = 0;
            for (int c = 1; c <= M; ++c)
                if (depth[static_cast<int64_t>(b) * R + c] >= 1 && anc[(static_cast<int64_t>(b) * R + c) * W + 1] == u)
                    kids[k++] = c;
            nkids = k;
        }
        __syncthreads();
        const int nk = nkids;
        bool moved = false;
        if (nk > 0) {
            const float *qr = q + b * qsb + static_cast<int64_t>(u) * qsr;
            int bd = 0;
            u128 sq = 0;
            for (int x = tid; x < V; x += kSampleThreads) sq += quantise(qr[x], bd);
            if (block_or(bd, &shflag)) { finish(TMV_ERR_INPUT, 0, 0); return; }
            const u128 SQ = block_sum_u128(sq, sh128);
            if (SQ == 0) { finish(TMV_ERR_INPUT, 0, 0); return; }
            for (int ci = 0; ci < nk; ++ci) {
                const int c = kids[ci];
                const int x = tokens[static_cast<int64_t>(b) * R + c];
                // W(x) and Wq(x) (any thread computes them; broadcast through LDS)
                __syncthreads();
                if (tid == 0) {
                    int bd2 = 0;
                    shx[0] = dist_at(cur, w, x, bd2);
                    shx[1] = quantise(qr[x], bd2);
                }
                __syncthreads();
                const uint64_t wx = shx[0], wqx = shx[1];
                const uint64_t U = tmv::philox_word(seed, stream, n++) >> 40;
                if (static_cast<u128>(U) * wqx * cur.S < (static_cast<u128>(wx) * SQ) << 24) {
                    if (tid == 0) pth[acc] = c;
                    ++acc;
                    u = c;
                    if (!load_p(c, cur)) { finish(TMV_ERR_INPUT, 0, 0); return; }
                    moved = true;
                    break;
                }
                // residual: W(y) <- max(0, W(y) SQ - Wq(y) S), renormalised
                u128 sn = 0;
                for (int y = tid; y < V; y += kSampleThreads) {
                    int bd3 = 0;
                    const u128 a = static_cast<u128>(dist_at(cur, w, y, bd3)) * SQ;
                    const u128 c2 = static_cast<u128>(quantise(qr[y], bd3)) * cur.S;
                    sn += a > c2 ? a - c2 : 0;
                }
                sn = block_sum_u128(sn, sh128);
                if (sn == 0) continue;          // empty residual: keep the distribution
                const int bl = tmv::bitlen_u128(sn);
                const int sh = bl > 48 ? bl - 48 : 0;
                // write the shifted residual; reading W(y) and writing w[y] happen in
                // the same thread for the same y, so the update is safe in place
                u128 s2 = 0;
                for (int y = tid; y < V; y += kSampleThreads) {
                    int bd3 = 0;
                    const u128 a = static_cast<u128>(dist_at(cur, w, y, bd3)) * SQ;
                    const u128 c2 = static_cast<u128>(quantise(qr[y], bd3)) * cur.S;
                    const uint64_t nv = static_cast<uint64_t>((a > c2 ? a - c2 : 0) >> sh);
                    w[y] = nv;
                    s2 += nv;
                }
                s2 = block_sum_u128(s2, sh128);
                cur.stored = true;
                cur.S = s2;
            }
            if (moved) continue;
        }
        // draw the bonus (no children) or the correction (all refused) from (W, S)
        const uint64_t word = tmv::philox_word(seed, stream, n++);
        const u128 t = (static_cast<u128>(word >> 32) * cur.S) >> 32;
        // contiguous segment per thread, exclusive scan of segment sums
        const int seg = (V + kSampleThreads - 1) / kSampleThreads;
        const int x0 = min(V, tid * seg), x1 = min(V, x0 + seg);
        u128 ssum = 0;
        int bd = 0;
        for (int x = x0; x < x1; ++x) ssum += dist_at(cur, w, x, bd);
        // inclusive scan of the segment sums inside the wave (shuffles up, 32-bit parts)
        const int lane = tid & (kWave - 1), wv = tid / kWave;
        u128 incl = ssum;
        for (int o = 1; o < kWave; o <<= 1) {
            u128 y = 0;
#pragma unroll
            for (int part = 0; part < 4; ++part) {
                const uint32_t v32 = static_cast<uint32_t>(incl >> (32 * part));
                y |= static_cast<u128>(static_cast<uint32_t>(__shfl_up(v32, o, kWave))) << (32 * part);
            }
            if (lane >= o) incl += y;
        }
        __syncthreads();
        if (lane == kWave - 1) sh128[wv] = incl;
        if (tid == 0) draw_tok = V - 1;
        __syncthreads();
        u128 before = 0;
        for (int w2 = 0; w2 < wv; ++w2) before += sh128[w2];
        const u128 excl = before + incl - ssum;
        // the thread whose segment holds the crossing point finds the token
        if (ssum > 0 && excl <= t && t < excl + ssum) {
            u128 cacc = excl;
            for (int x = x0; x < x1; ++x) {
                cacc += dist_at(cur, w, x, bd);
                if (cacc > t) { draw_tok = x; break; }
            }
        }
        __syncthreads();
        finish(TMV_OK, acc, draw_tok);
        return;
    }
}

}  // namespace

extern "C" size_t tmv_tree_accept_workspace(int mode, int B, int M_max, int V)
{
    if (B <= 0 || M_max < 0 || V <= 0) return 256;
    if (mode == TMV_ACCEPT_GREEDY) {
        const int nchunk = (V + kScanChunk - 1) / kScanChunk;
        return static_cast<size_t>(B) * (M_max + 1) * nchunk * sizeof(uint64_t) + 256;
    }
    return static_cast<size_t>(B) * V * sizeof(uint64_t) + 256;
}

extern "C" int tmv_tree_accept(int mode, int B, int M_max, int D_max, int V,
                               const int32_t *tokens, int row_dtype, const void *teacher,
                               int64_t t_stride_b, int64_t t_stride_row,
                               const float *draft_q, int64_t q_stride_b, int64_t q_stride_row,
                               uint64_t seed, uint64_t step,
                               const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                               int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (mode != TMV_ACCEPT_GREEDY && mode != TMV_ACCEPT_SAMPLE) return TMV_ERR_ARG;
    if (B < 0 || M_max < 0 || M_max > 128 || D_max < 0 || D_max > 128 || V < 1) return TMV_ERR_ARG;
    if (t_stride_b < 0 || t_stride_row < 0) return TMV_ERR_ARG;
    if (B == 0) return TMV_OK;
    if (!tokens || !teacher || !n_nodes || !anc || !depth || !status || !accept_len || !next_token)
        return TMV_ERR_ARG;
    if (D_max > 0 && !path) return TMV_ERR_ARG;
    if (!workspace || workspace_bytes < tmv_tree_accept_workspace(mode, B, M_max, V)) return TMV_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return TMV_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);

    if (mode == TMV_ACCEPT_GREEDY) {
        if (row_dtype != TMV_F32 && row_dtype != TMV_BF16) return TMV_ERR_ARG;
        const int nchunk = (V + kScanChunk - 1) / kScanChunk;
        const int64_t blocks = static_cast<int64_t>(B) * (M_max + 1) * nchunk;
        if (blocks > 0x7fffffff) return TMV_ERR_ARG;
        uint64_t *keys = reinterpret_cast<uint64_t *>(ws);
        if (row_dtype == TMV_F32)
            hipLaunchKernelGGL(greedy_scan_kernel<TMV_F32>, dim3(static_cast<unsigned>(blocks)), dim3(kScanThreads), 0, s,
                               M_max, V, nchunk, teacher, t_stride_b, t_stride_row, n_nodes, depth, status, keys);
        else
            hipLaunchKernelGGL(greedy_scan_kernel<TMV_BF16>, dim3(static_cast<unsigned>(blocks)), dim3(kScanThreads), 0, s,
                               M_max, V, nchunk, teacher, t_stride_b, t_stride_row, n_nodes, depth, status, keys);
        hipLaunchKernelGGL(greedy_select_kernel, dim3(B), dim3(kScanThreads), 0, s, M_max, D_max, V, nchunk, tokens,
                           n_nodes, anc, depth, status, accept_len, path, next_token, keys);
        return tmv_host::launch_status(hipGetLastError());
    }
    if (row_dtype != TMV_F32 || !draft_q || q_stride_b < 0 || q_stride_row < 0) return TMV_ERR_ARG;
    hipLaunchKernelGGL(sample_walk_kernel, dim3(B), dim3(kSampleThreads), 0, s, M_max, D_max, V, tokens,
                       static_cast<const float *>(teacher), t_stride_b, t_stride_row, draft_q, q_stride_b,
                       q_stride_row, seed, step, n_nodes, anc, depth, status, accept_len, path, next_token,
                       reinterpret_cast<uint64_t *>(ws));
    return tmv_host::launch_status(hipGetLastError());
}
